"""bench.py's output contract: one JSON line with the metric, the whole-step
throughput, the roofline of the dominant kernel and the CPU baseline, run in
a child process on the small Erdos-Renyi workload (fp32, 1,000 nodes)."""
import json
import os
import subprocess
import sys

import pytest

from tests.gpu_util import note

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_json_line():
    note("bench.py on gt_er1k_h4d32_f32")
    r = subprocess.run([sys.executable, "bench.py", "--workload", "gt_er1k_h4d32_f32",
                        "--steps", "3", "--warmup", "1", "--cpu-seconds", "1", "--step-times",
                        "--probe-gib", "0.5", "--extra", "gt_er1k_h4d32_f32"],
                       cwd=ROOT, capture_output=True, text=True, timeout=240)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1, r.stdout[-2000:]
    d = json.loads(lines[0])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
              "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
              "roofline", "cpu_baseline"):
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1
    assert d["higher_is_better"] is True and d["value"] > 0 and d["ms_per_step"] > 0
    assert d["config"]["workload"] == "gt_er1k_h4d32_f32"
    # value is E * H per step time; both are printed to 4 decimals, so the
    # step time carries up to 5e-5 ms of rounding
    c = d["config"]
    ms = d["ms_per_step"]
    assert abs(d["value"] - c["edges"] * c["heads"] / (ms * 1e-3) / 1e9) \
        <= d["value"] * (5e-5 / ms + 1e-6) + 1e-4
    roof = d["roofline"]
    for k in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert k in roof, k
    assert roof["bound"] == "hbm" and roof["unit"] == "GB/s" and roof["peak"] == 8000.0
    assert abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-3
    # a fraction above 1 is only possible if caches served modelled gathers,
    # and the line must say so
    assert (roof["frac"] > 1) == roof["cache_served"]
    assert (d["step_model"]["frac"] > 1) == d["step_model"]["cache_served"]
    # (ms_per_step is printed to 4 decimals: up to 5e-5 ms of rounding)
    assert abs(d["step_model"]["gbs"] - d["step_model"]["bytes"] / (ms * 1e-3) / 1e9) \
        <= d["step_model"]["gbs"] * (5e-5 / ms + 1e-3) + 0.1
    hc = d["hbm_ceiling"]
    assert 0 < hc["stream_read_gbs"] and 0 < hc["gather_gbs"] and hc["spec_gbs"] == 8000.0
    assert roof["frac_of_ceiling"] > 0
    assert d["warm"]["ms_per_step"] > 0 and d["warm"]["value"] > 0
    mem = d["memory"]
    assert mem["inputs_bytes"] == 3 * 1000 * 4 * 32 * 4      # Q, K, V fp32
    assert mem["workspace_bytes"]["fwd"] >= 0 and mem["plan_bytes"] > 0
    cf = d["configs"]["gt_er1k_h4d32_f32"]
    assert cf["ms_per_step"] > 0 and cf["value"] > 0 and cf["edges"] == c["edges"]
    for kind in ("warm", "cold"):          # each step timed alone, median and minimum
        st = d["steps_ms"][kind]
        assert 0 < st["min"] <= st["median"] and st["reps"] == 3 and st["value"] > 0
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["cores"] >= 1 and cb["sample"]
    assert cb["cpu"]


def test_bench_refuses_several_gpus():
    r = subprocess.run([sys.executable, "bench.py", "--gpus", "2"], cwd=ROOT,
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0 and "one GPU" in r.stderr


def test_trace_only_brackets_one_kernel():
    """The timing trace records every launch, or with trace_only(name) just the
    launches of that kernel, and tracing changes no result."""
    import numpy as np
    import torch

    from sparse_graph_attention_csr_amd import binding as B
    from sparse_graph_attention_csr_amd import inputs as I
    from tests.gpu_util import Runner

    rng = np.random.default_rng(3)
    rp, ci = I.random_csr(300, 9, rng, heavy_rows=1, heavy_deg=900)
    r = Runner(rp, ci, device=torch.device("cuda:0"), chunk=128)
    q, k, v, do = (torch.from_numpy(I.normal_tensor(rng, (300, 2, 32), I.F32)).cuda()
                   for _ in range(4))
    ref_out, ref_lse = r.gt_fwd(q, k, v)
    ref = r.gt_bwd(q, k, v, ref_out, ref_lse, do)

    def traced(only):
        B.trace_clear()
        B.trace_only(only)
        B.trace_enable(True)
        try:
            out, lse = r.gt_fwd(q, k, v)
            grads = r.gt_bwd(q, k, v, out, lse, do)
            torch.cuda.synchronize()
        finally:
            B.trace_enable(False)
            B.trace_only(None)
        recs = B.trace_read()
        B.trace_clear()
        for a, b in zip((out, lse) + grads, (ref_out, ref_lse) + ref):
            assert torch.equal(a, b)
        return recs

    every = traced(None)
    names = [n for n, _ in every]
    assert {"gt_fwd_rows", "gt_bwd_cols", "gt_bwd_rows"} <= set(names)
    assert all(ms >= 0 for _, ms in every)
    one = traced("gt_bwd_cols")
    assert [n for n, _ in one] == ["gt_bwd_cols"] * names.count("gt_bwd_cols")
    assert traced("no_such_kernel") == []


def test_probes_load_and_leave_the_sink_alone():
    """The bandwidth probes run on ones-filled buffers (every folded word is
    0, never the sink constant) and skip row indices outside the table."""
    import torch

    from sparse_graph_attention_csr_amd import binding as B
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    buf = torch.ones(1 << 20, dtype=torch.int32, device="cuda")
    B.probe_read(buf, sink, 64)
    table = torch.ones(1000, 256, dtype=torch.int32, device="cuda")    # 1 KiB rows
    idx = torch.tensor([0, 999, 1000, 5000, -1, 3] * 50, dtype=torch.int32, device="cuda")
    B.probe_gather(table, idx, sink)
    torch.cuda.synchronize()
    assert int(sink.abs().sum()) == 0
    with pytest.raises(B.SgatError):
        B.probe_gather(torch.ones(10, 3, dtype=torch.int32, device="cuda"), idx, sink)  # 12-byte rows
