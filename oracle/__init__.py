"""fp64 CPU oracle for fused graph attention (TEST INFRASTRUCTURE ONLY).

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The product path (the HIP library and its
Python binding) never loads it, and it shares no code with them.

``oracle.c`` computes the plain definition of Graph Transformer and GATv2
attention over a CSR neighbourhood in fp64 (forward and the softmax-Jacobian
backward), and of min/max reduction aggregation (forward with its winning
edges, and the backward that routes each gradient to its winner); ``plan_spec.py`` is an independent numpy statement of the integer
preprocessing arrays (work lists, transposed CSR, 16x16 tiles).

Inputs may be numpy float32, float64 or uint16 (bf16 bit patterns); they are
widened exactly to fp64 inside the C code.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
# SGAT_ORACLE_LIBRARY selects another build (the sanitizer build, see build())
_LIB = os.environ.get("SGAT_ORACLE_LIBRARY") or os.path.join(_HERE, "liboracle.so")
_SAN_LIB = os.path.join(_HERE, "liboracle_san.so")

_DT = {np.dtype(np.float32): 0, np.dtype(np.uint16): 1, np.dtype(np.float64): 2}


def build(force: bool = True, sanitize: bool = False) -> str:
    """Compile oracle.c with gcc (-O2, OpenMP, IEEE semantics kept). With
    sanitize, build liboracle_san.so instead with clang's AddressSanitizer and
    UndefinedBehaviorSanitizer (the runtime the library's sanitizer build
    uses, so both can share one process)."""
    if sanitize:
        llvm = "/opt/rocm/llvm"
        tmp = _SAN_LIB + ".tmp"
        subprocess.check_call([f"{llvm}/bin/clang", "-O1", "-g", "-fno-omit-frame-pointer",
                               "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                               "-fopenmp", "-fPIC", "-shared", "-std=c99", "-Wall", "-Wextra",
                               f"-Wl,-rpath,{llvm}/lib", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _SAN_LIB)
        return _SAN_LIB
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99",
                               "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        i64, i32, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
        dbl = ctypes.c_double
        lib.oracle_num_threads.restype = i32
        lib.oracle_gt_fwd.argtypes = [i64, vp, vp, i32, i32, i32, vp, vp, vp, i64, vp, vp, vp]
        lib.oracle_gat_fwd.argtypes = [i64, vp, vp, i32, i32, i32, vp, vp, vp, dbl, i64, vp, vp, vp]
        lib.oracle_gt_bwd.argtypes = [i64, vp, vp, i32, i32, i32, vp, vp, vp, vp,
                                      i64, vp, vp, i64, vp, vp, vp]
        lib.oracle_gat_bwd.argtypes = [i64, vp, vp, i32, i32, i32, vp, vp, vp, dbl, vp,
                                       i64, vp, vp, i64, vp, vp, vp]
        lib.oracle_reduce_fwd.argtypes = [i64, vp, vp, i32, i32, i32, vp, i64, vp, vp, vp]
        lib.oracle_reduce_bwd.argtypes = [i64, vp, vp, i32, i32, vp, vp, vp]
        for f in (lib.oracle_gt_fwd, lib.oracle_gat_fwd, lib.oracle_gt_bwd, lib.oracle_gat_bwd,
                  lib.oracle_reduce_fwd, lib.oracle_reduce_bwd):
            f.restype = i32
        _lib = lib
    return _lib


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _features(*arrs):
    dts = {a.dtype for a in arrs}
    if len(dts) != 1:
        raise TypeError(f"feature arrays must share one dtype, got {dts}")
    dt = dts.pop()
    if dt not in _DT:
        raise TypeError(f"unsupported dtype {dt}")
    if arrs[0].ndim != 3:
        raise ValueError("features must be [N, H, D]")
    return [np.ascontiguousarray(a) for a in arrs], _DT[dt]


def _graph(rowptr, colidx):
    return (np.ascontiguousarray(rowptr, dtype=np.int64),
            np.ascontiguousarray(colidx, dtype=np.int32))


def _sel(rows):
    if rows is None:
        return None, 0
    r = np.ascontiguousarray(rows, dtype=np.int64)
    return r, r.size


def _check(rc, name):
    if rc != 0:
        raise RuntimeError(f"{name} failed with code {rc}")


def gt_fwd(rowptr, colidx, q, k, v, rows=None):
    """Graph Transformer forward: (out [n|len(rows), H, D], lse [.., H]) in fp64."""
    rowptr, colidx = _graph(rowptr, colidx)
    (q, k, v), dt = _features(q, k, v)
    n, H, D = q.shape
    sel, ns = _sel(rows)
    cnt = ns if sel is not None else n
    out = np.empty((cnt, H, D), dtype=np.float64)
    lse = np.empty((cnt, H), dtype=np.float64)
    _check(_load().oracle_gt_fwd(n, _p(rowptr), _p(colidx), H, D, dt, _p(q), _p(k), _p(v),
                                 ns, _p(sel), _p(out), _p(lse)), "oracle_gt_fwd")
    return out, lse


def gat_fwd(rowptr, colidx, xs, xt, a, slope=0.2, rows=None):
    """GATv2 forward: (out, lse) in fp64. ``a`` is [H, D] (any float type)."""
    rowptr, colidx = _graph(rowptr, colidx)
    (xs, xt), dt = _features(xs, xt)
    n, H, D = xs.shape
    a = np.ascontiguousarray(a, dtype=np.float64).reshape(H, D)
    sel, ns = _sel(rows)
    cnt = ns if sel is not None else n
    out = np.empty((cnt, H, D), dtype=np.float64)
    lse = np.empty((cnt, H), dtype=np.float64)
    _check(_load().oracle_gat_fwd(n, _p(rowptr), _p(colidx), H, D, dt, _p(xs), _p(xt), _p(a),
                                  float(slope), ns, _p(sel), _p(out), _p(lse)), "oracle_gat_fwd")
    return out, lse


def gt_bwd(rowptr, colidx, q, k, v, dout, dst_rows=None, src_rows=None):
    """Graph Transformer backward of L = sum(out * dout): (dQ, dK, dV) in fp64.

    dQ holds the rows ``dst_rows`` (all if None); dK and dV hold ``src_rows``.
    """
    rowptr, colidx = _graph(rowptr, colidx)
    (q, k, v, dout), dt = _features(q, k, v, dout)
    n, H, D = q.shape
    sd, nd = _sel(dst_rows)
    ss, nss = _sel(src_rows)
    dq = np.empty((nd if sd is not None else n, H, D), dtype=np.float64)
    dk = np.empty((nss if ss is not None else n, H, D), dtype=np.float64)
    dv = np.empty_like(dk)
    _check(_load().oracle_gt_bwd(n, _p(rowptr), _p(colidx), H, D, dt, _p(q), _p(k), _p(v),
                                 _p(dout), nd, _p(sd), _p(dq), nss, _p(ss), _p(dk), _p(dv)),
           "oracle_gt_bwd")
    return dq, dk, dv


def gat_bwd(rowptr, colidx, xs, xt, a, dout, slope=0.2, dst_rows=None, src_rows=None):
    """GATv2 backward of L = sum(out * dout): (dXs, dXt, da) in fp64."""
    rowptr, colidx = _graph(rowptr, colidx)
    (xs, xt, dout), dt = _features(xs, xt, dout)
    n, H, D = xs.shape
    a = np.ascontiguousarray(a, dtype=np.float64).reshape(H, D)
    sd, nd = _sel(dst_rows)
    ss, nss = _sel(src_rows)
    dxs = np.empty((nd if sd is not None else n, H, D), dtype=np.float64)
    dxt = np.empty((nss if ss is not None else n, H, D), dtype=np.float64)
    da = np.empty((H, D), dtype=np.float64)
    _check(_load().oracle_gat_bwd(n, _p(rowptr), _p(colidx), H, D, dt, _p(xs), _p(xt), _p(a),
                                  float(slope), _p(dout), nd, _p(sd), _p(dxs), nss, _p(ss),
                                  _p(dxt), _p(da)), "oracle_gat_bwd")
    return dxs, dxt, da


_OPS = {"min": 0, "max": 1}


def _features2(x):
    x = np.ascontiguousarray(x)
    if x.dtype not in _DT:
        raise TypeError(f"unsupported dtype {x.dtype}")
    if x.ndim != 2:
        raise ValueError("reduction features must be [N, F]")
    return x, _DT[x.dtype]


def reduce_fwd(rowptr, colidx, x, op="min", rows=None):
    """Min or max aggregation of the source rows x [N, F] over each row's
    in-edges: (out fp64, arg int64), both [rows or N, F]. arg holds the CSR
    position of the winning edge (the first one on ties), -1 for empty rows,
    whose out is 0."""
    rowptr, colidx = _graph(rowptr, colidx)
    x, dt = _features2(x)
    n, F = x.shape
    s, ns = _sel(rows)
    cnt = ns if s is not None else n
    out = np.empty((cnt, F), dtype=np.float64)
    arg = np.empty((cnt, F), dtype=np.int64)
    _check(_load().oracle_reduce_fwd(n, _p(rowptr), _p(colidx), F, dt, _OPS[op], _p(x), ns,
                                     _p(s), _p(out), _p(arg)), "oracle_reduce_fwd")
    return out, arg


def reduce_bwd(rowptr, colidx, arg, dout):
    """Backward of L = sum(out * dout) for the aggregation whose winners are
    ``arg`` [N, F] (as reduce_fwd returns over all rows): dX fp64 [N, F]."""
    rowptr, colidx = _graph(rowptr, colidx)
    dout, dt = _features2(dout)
    n, F = dout.shape
    arg = np.ascontiguousarray(arg, dtype=np.int64)
    if arg.shape != (n, F):
        raise ValueError("arg must be [N, F]")
    dx = np.empty((n, F), dtype=np.float64)
    _check(_load().oracle_reduce_bwd(n, _p(rowptr), _p(colidx), F, dt, _p(arg), _p(dout),
                                     _p(dx)), "oracle_reduce_bwd")
    return dx
