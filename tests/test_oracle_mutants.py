"""Planted mistakes in the oracle must be caught by its pins (CPU only).

Each mutant is oracle.c with one plausible error: a dropped term or scale, a
wrong sign, a transposed operand or index, a wrong LeakyReLU branch, a wrong
empty-row convention, a wrong tie rule or gradient route of the min/max
aggregation. It is compiled into a temporary directory and run
through the pin tests of test_oracle.py and test_oracle_reduce.py; every
mutant must fail at least one.
The oracle under test/oracle.c itself is never modified.
"""
import importlib.util
import os
import subprocess

import pytest

from tests import test_oracle as T
from tests import test_oracle_reduce as TR

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

# (name, exact text in oracle.c, replacement); each text occurs exactly once
MUTANTS = [
    ("gt score without 1/sqrt(D)", "return s / sqrt((double)D);", "return s;"),
    ("gt score ignores the head", "s += ld(Q, dt, (i * H + h) * D + d) * ld(K, dt, (j * H + h) * D + d);",
     "s += ld(Q, dt, (i * H) * D + d) * ld(K, dt, (j * H + h) * D + d);"),
    ("lse without the max", "return m + log(l);", "return log(l);"),
    ("output aggregates keys", "o[d] += s[t] * ld(C, dt, (j * H + h) * D + d);",
     "o[d] += s[t] * ld(B, dt, (j * H + h) * D + d);"),
    ("empty-row lse 0", "if (deg == 0) { lse[r * H + h] = -INFINITY; continue; }",
     "if (deg == 0) { lse[r * H + h] = 0.0; continue; }"),
    ("gatv2 score reads Xs for the neighbour",
     "double z = ld(Xs, dt, (i * H + h) * D + d) + ld(Xt, dt, (j * H + h) * D + d);\n        s += a[h * D + d] * lrelu(z, slope);",
     "double z = ld(Xs, dt, (i * H + h) * D + d) + ld(Xs, dt, (j * H + h) * D + d);\n        s += a[h * D + d] * lrelu(z, slope);"),
    ("leaky relu slope dropped", "static double lrelu(double z, double slope) { return z > 0.0 ? z : slope * z; }",
     "static double lrelu(double z, double slope) { (void)slope; return z > 0.0 ? z : 0.0 * z; }"),
    ("leaky relu derivative 0 below zero",
     "static double lrelu_grad(double z, double slope) { return z > 0.0 ? 1.0 : slope; }",
     "static double lrelu_grad(double z, double slope) { (void)slope; return z > 0.0 ? 1.0 : 0.0; }"),
    ("softmax jacobian sign", "dS[(b + t) * H + h] = alpha[(b + t) * H + h] * (dp[t] - c);",
     "dS[(b + t) * H + h] = alpha[(b + t) * H + h] * (c - dp[t]);"),
    ("softmax jacobian drops the mean", "dS[(b + t) * H + h] = alpha[(b + t) * H + h] * (dp[t] - c);",
     "dS[(b + t) * H + h] = alpha[(b + t) * H + h] * dp[t];"),
    ("dQ from Q instead of K", "g[d] += dS[e * H + h] * ld(K, dtype, (j * H + h) * D + d) * inv;",
     "g[d] += dS[e * H + h] * ld(Q, dtype, (j * H + h) * D + d) * inv;"),
    ("dK from the source's Q", "gk[d] += dS[e * H + h] * ld(Q, dtype, (i * H + h) * D + d) * inv;",
     "gk[d] += dS[e * H + h] * ld(Q, dtype, (j * H + h) * D + d) * inv;"),
    ("dV weighted by dS", "gv[d] += alpha[e * H + h] * ld(dout, dtype, (i * H + h) * D + d);",
     "gv[d] += dS[e * H + h] * ld(dout, dtype, (i * H + h) * D + d);"),
    ("dK without 1/sqrt(D)", "gk[d] += dS[e * H + h] * ld(Q, dtype, (i * H + h) * D + d) * inv;",
     "gk[d] += dS[e * H + h] * ld(Q, dtype, (i * H + h) * D + d);"),
    ("gatv2 dXt drops the value term",
     "g[d] += dE[e * H + h] * a[h * D + d] * lrelu_grad(z, slope)\n                          + alpha[e * H + h] * ld(dout, dtype, (i * H + h) * D + d);",
     "g[d] += dE[e * H + h] * a[h * D + d] * lrelu_grad(z, slope);"),
    ("gatv2 da uses the derivative", "p[h * D + d] += dE[e * H + h] * lrelu(z, slope);",
     "p[h * D + d] += dE[e * H + h] * lrelu_grad(z, slope);"),
    ("gatv2 dXs misses a", "g[d] += dE[e * H + h] * a[h * D + d] * lrelu_grad(z, slope);\n",
     "g[d] += dE[e * H + h] * lrelu_grad(z, slope);\n"),
    ("transposed CSR stores rows for edge ids", "eid[fill[colidx[e]]++] = e;",
     "eid[fill[colidx[e]]++] = e > 0 ? e - 1 : e;"),
    ("reduction ties go to the last edge", "int better = op == 0 ? x < v[f] : x > v[f];",
     "int better = op == 0 ? x <= v[f] : x >= v[f];"),
    ("max uses the min comparison", "int better = op == 0 ? x < v[f] : x > v[f];",
     "int better = x < v[f];"),
    ("empty reduction row gives +inf", "{ v[f] = 0.0; w[f] = -1; }",
     "{ v[f] = INFINITY; w[f] = -1; }"),
    ("first edge not taken unconditionally", "if (w[f] < 0 || better) { v[f] = x; w[f] = e; }",
     "if (better) { v[f] = x; w[f] = e; }"),
    ("reduction gradient routed to the destination",
     "dX[(int64_t)colidx[e] * F + f] += ld(dout, dtype, i * F + f);",
     "dX[i * F + f] += ld(dout, dtype, i * F + f);"),
    ("reduction gradient reads the source's dout",
     "dX[(int64_t)colidx[e] * F + f] += ld(dout, dtype, i * F + f);",
     "dX[(int64_t)colidx[e] * F + f] += ld(dout, dtype, (int64_t)colidx[e] * F + f);"),
]

# pins run against every mutant: (test function, keyword arguments)
PINS = [
    (T.test_gt_golden_closed_form, {}),
    (T.test_gat_golden_closed_form, {}),
    (T.test_gt_matches_masked_dense, {"case": "multigraph_empty"}),
    (T.test_gat_matches_masked_dense, {"case": "multigraph_empty"}),
    (T.test_gt_backward_matches_dense_autograd, {}),
    (T.test_gat_backward_matches_dense_autograd, {}),
    (T.test_gt_backward_finite_differences, {}),
    (T.test_gat_backward_finite_differences, {}),
    (T.test_empty_rows, {}),
    (TR.test_reduce_golden_ties, {"op": "min"}),
    (TR.test_reduce_golden_ties, {"op": "max"}),
    (TR.test_reduce_matches_numpy_first_occurrence, {"op": "min", "dtype": "f64"}),
    (TR.test_reduce_matches_numpy_first_occurrence, {"op": "max", "dtype": "f64"}),
    (TR.test_reduce_backward_matches_dense_autograd, {"op": "min"}),
]


def load_mutant(tmp_path, k, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation text must occur once: {old!r}"
    mdir = tmp_path / f"m{k}"
    mdir.mkdir()
    c = mdir / "oracle.c"
    c.write_text(src.replace(old, new))
    so = mdir / "liboracle.so"
    subprocess.check_call(["gcc", "-O1", "-fopenmp", "-fPIC", "-shared", "-std=c99", "-o",
                           str(so), str(c), "-lm"])
    spec = importlib.util.spec_from_file_location(f"oracle_mutant_{k}",
                                                  os.path.join(ROOT, "oracle", "__init__.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    mod._LIB = str(so)
    mod._lib = None
    return mod


def test_unmutated_oracle_passes_the_battery(oracle_mod):
    for fn, kw in PINS:
        fn(oracle_mod, **kw)


@pytest.mark.parametrize("k", range(len(MUTANTS)), ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, k):
    name, old, new = MUTANTS[k]
    mod = load_mutant(tmp_path, k, old, new)
    caught = []
    for fn, kw in PINS:
        try:
            fn(mod, **kw)
        except (AssertionError, RuntimeError, ValueError, FloatingPointError):
            caught.append(fn.__name__)
    assert caught, f"mutant '{name}' passed every pin"
