"""Thin Python binding of libsgattn.so (ctypes).

Argument marshalling only: every step of the computation runs in the HIP
library. torch tensors supply device memory and the stream; the functions
``gt_fwd``, ``gt_bwd``, ``gat_fwd``, ``gat_bwd``, ``reduce_fwd`` and
``reduce_bwd`` mirror the C entry points
of the same names in include/sgattn.h, and raise :class:`SgatError` on a
non-zero status. There is no fallback: if the library is missing, loading it
raises.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

# SGAT_LIBRARY selects another build of the same library (the sanitizer build)
_LIB_PATH = os.environ.get("SGAT_LIBRARY") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "libsgattn.so")

F32, BF16 = 0, 1
OP_GT_FWD, OP_GT_BWD, OP_GAT_FWD, OP_GAT_BWD, OP_REDUCE_FWD, OP_REDUCE_BWD = range(6)
REDUCE_MIN, REDUCE_MAX = 0, 1
REDUCE_OPS = {"min": REDUCE_MIN, "max": REDUCE_MAX}

(ARR_ROW_ITEMS, ARR_ROW_SPLITS, ARR_COLPTR, ARR_ROWIDX, ARR_COL_ITEMS, ARR_COL_SPLITS,
 ARR_TILE_ROWPTR, ARR_TILE_COL, ARR_TILE_MASK, ARR_RES_ROWPTR, ARR_RES_COLIDX,
 ARR_TILE_ROW, ARR_TILE_COLPTR, ARR_TILE_BYCOL, ARR_RES_COLPTR, ARR_RES_ROWIDX,
 ARR_COL_EDGE, ARR_RES_COL_EDGE, ARR_ROW_TPOS, ARR_RES_ROW, ARR_RES_COLSRC,
 ARR_TILE_ROW_BYCOL) = range(22)

STATUS = {0: "OK", 1: "INVALID_ARGUMENT", 2: "INVALID_CSR", 3: "WORKSPACE_TOO_SMALL",
          4: "PLAN_MISMATCH", 5: "HIP_ERROR", 6: "NOT_UPLOADED", 7: "OUT_OF_HOST_MEMORY",
          8: "UNSUPPORTED", 9: "SCRATCH_LIMIT"}

# bytes of the static device scratch gt_fwd_noalloc uses (SGAT_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 32 << 20

WORK_ITEM_DTYPE = np.dtype([("begin", "<i8"), ("len", "<i4"), ("row", "<i4"),
                            ("slot", "<i4"), ("flags", "<i4")])
SPLIT_DTYPE = np.dtype([("row", "<i4"), ("first_slot", "<i4"), ("nslots", "<i4"),
                        ("reserved", "<i4")])
ARRAY_DTYPES = {
    ARR_ROW_ITEMS: WORK_ITEM_DTYPE, ARR_ROW_SPLITS: SPLIT_DTYPE,
    ARR_COLPTR: np.dtype("<i8"), ARR_ROWIDX: np.dtype("<i4"),
    ARR_COL_ITEMS: WORK_ITEM_DTYPE, ARR_COL_SPLITS: SPLIT_DTYPE,
    ARR_TILE_ROWPTR: np.dtype("<i8"), ARR_TILE_COL: np.dtype("<i4"),
    ARR_TILE_MASK: np.dtype("<u2"), ARR_RES_ROWPTR: np.dtype("<i8"),
    ARR_RES_COLIDX: np.dtype("<i4"), ARR_TILE_ROW: np.dtype("<i4"),
    ARR_TILE_COLPTR: np.dtype("<i8"), ARR_TILE_BYCOL: np.dtype("<i4"),
    ARR_RES_COLPTR: np.dtype("<i8"), ARR_RES_ROWIDX: np.dtype("<i4"),
    ARR_COL_EDGE: np.dtype("<i4"), ARR_RES_COL_EDGE: np.dtype("<i4"),
    ARR_ROW_TPOS: np.dtype("<i4"), ARR_RES_ROW: np.dtype("<i4"), ARR_RES_COLSRC: np.dtype("<i4"),
    ARR_TILE_ROW_BYCOL: np.dtype("<i4"),
}


class SgatError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: {STATUS.get(status, status)} ({status})")


class PlanOpts(ctypes.Structure):
    _fields_ = [("chunk", ctypes.c_int64), ("tile_min_nnz", ctypes.c_int32),
                ("block_sparse", ctypes.c_int32), ("locality", ctypes.c_int32),
                ("edge_order", ctypes.c_int32)]


class PlanStats(ctypes.Structure):
    _fields_ = [(name, ctypes.c_int64) for name in (
        "n", "nnz", "chunk", "max_in_degree", "max_out_degree",
        "row_items", "row_splits", "row_slots", "col_items", "col_splits", "col_slots",
        "tiles", "tile_edges", "residual_edges", "device_bytes")]


_lib = None

# name -> (restype, argtypes); kept in the order of include/sgattn.h
_i64, _i32, _vp, _sz, _f = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_float
_SIGS = {
    "sgat_plan_create": (_i32, [_i64, _i64, _vp, _vp, ctypes.POINTER(PlanOpts), ctypes.POINTER(_vp)]),
    "sgat_plan_device_bytes": (_i32, [_vp, ctypes.POINTER(_sz)]),
    "sgat_plan_upload": (_i32, [_vp, _vp, _sz, _vp]),
    "sgat_plan_stats_get": (_i32, [_vp, ctypes.POINTER(PlanStats)]),
    "sgat_plan_array_bytes": (_i32, [_vp, _i32, ctypes.POINTER(_sz)]),
    "sgat_plan_export": (_i32, [_vp, _i32, _vp, _sz]),
    "sgat_plan_destroy": (None, [_vp]),
    "sgat_workspace_bytes": (_i32, [_vp, _i32, _i32, _i32, _i32, ctypes.POINTER(_sz)]),
    "gt_fwd": (_i32, [_vp, _i64, _i64, _vp, _vp, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp,
                      _vp, _sz, _i32, _vp]),
    "gt_fwd_noalloc": (_i32, [_vp, _i64, _i64, _vp, _vp, _i32, _i32, _i32, _vp, _vp, _vp, _vp,
                              _vp, _i32, _vp]),
    "gt_bwd": (_i32, [_vp, _i64, _i64, _vp, _vp, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp,
                      _vp, _vp, _vp, _vp, _sz, _i32, _vp]),
    "gat_fwd": (_i32, [_vp, _i64, _i64, _vp, _vp, _i32, _i32, _i32, _vp, _vp, _vp, _f, _vp, _vp,
                       _vp, _sz, _vp]),
    "gat_bwd": (_i32, [_vp, _i64, _i64, _vp, _vp, _i32, _i32, _i32, _vp, _vp, _vp, _f, _vp, _vp,
                       _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "reduce_fwd": (_i32, [_vp, _i64, _i64, _vp, _vp, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _sz,
                          _vp]),
    "reduce_bwd": (_i32, [_vp, _i64, _i64, _vp, _vp, _i32, _i32, _vp, _vp, _vp, _vp, _sz, _vp]),
    "sgat_status_string": (ctypes.c_char_p, [_i32]),
    "sgat_probe_read": (_i32, [_vp, _sz, _vp, _i32, _vp]),
    "sgat_probe_gather": (_i32, [_vp, _i64, _i32, _vp, _i64, _vp, _vp]),
    "sgat_trace_enable": (_i32, [_i32]),
    "sgat_trace_only": (_i32, [ctypes.c_char_p]),
    "sgat_trace_clear": (_i32, []),
    "sgat_trace_count": (_i32, []),
    "sgat_trace_get": (_i32, [_i32, ctypes.c_char_p, _sz, ctypes.POINTER(_f)]),
}


def library_path() -> str:
    return _LIB_PATH


def lib() -> ctypes.CDLL:
    """The loaded libsgattn.so. Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(
                f"libsgattn.so not found at {_LIB_PATH}; build it with "
                "`python -m sparse_graph_attention_csr_amd.build` (no fallback exists)")
        L = ctypes.CDLL(_LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _check(fn: str, rc: int):
    if rc != 0:
        raise SgatError(fn, rc)


def status_string(st: int) -> str:
    return lib().sgat_status_string(st).decode()


# ---------------------------------------------------------------------------
# tensor marshalling
# ---------------------------------------------------------------------------

def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _ptr(t):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _stream(stream):
    import torch
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _shape(t):
    if t.dim() != 3:
        raise ValueError("feature tensors are [N, H, D]")
    return t.shape


def _expect(name, t, shape, dtype, device):
    """The C ABI receives bare pointers and cannot check sizes, so every tensor
    argument is checked here: shape, dtype, device and contiguity."""
    if t is None:
        raise ValueError(f"{name} is required")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _check_call(plan, rowptr, colidx, ws, lead, name="q"):
    """Common checks: the lead tensor is on a GPU and has the plan's n rows;
    the graph arrays are the plan's device CSR; the workspace is on the GPU."""
    import torch
    dev = lead.device
    if lead.shape[0] != plan.n:
        raise ValueError(f"{name} has {lead.shape[0]} rows, the plan {plan.n}")
    if dev.type != "cuda":
        raise ValueError(f"{name} is on {dev}: the library runs on the GPU")
    _expect("rowptr", rowptr, (plan.n + 1,), torch.int64, dev)
    _expect("colidx", colidx, (plan.nnz,), torch.int32, dev)
    if ws is not None and (ws.device != dev or not ws.is_contiguous()):
        raise ValueError("the workspace must be a contiguous tensor on the same GPU")
    return dev


def _ws_bytes(ws):
    return 0 if ws is None else ws.numel() * ws.element_size()


# ---------------------------------------------------------------------------
# plan
# ---------------------------------------------------------------------------

class Plan:
    """Host plan of one CSR graph (sgat_plan_create / _upload / _destroy)."""

    def __init__(self, rowptr, colidx, chunk: int = 0, tile_min_nnz: int = 0,
                 block_sparse: bool = False, locality: bool = False, edge_order: int = 0):
        rowptr = np.ascontiguousarray(rowptr, dtype=np.int64)
        colidx = np.ascontiguousarray(colidx, dtype=np.int32)
        self.n = int(rowptr.size - 1)
        self.nnz = int(colidx.size)
        self.edge_order = int(edge_order)
        opts = PlanOpts(int(chunk), int(tile_min_nnz), int(bool(block_sparse)),
                        int(bool(locality)), int(edge_order))
        h = ctypes.c_void_p()
        _check("sgat_plan_create",
               lib().sgat_plan_create(self.n, self.nnz, rowptr.ctypes.data, colidx.ctypes.data,
                                      ctypes.byref(opts), ctypes.byref(h)))
        self._h = h
        self._dev = None

    @property
    def handle(self):
        return self._h

    def close(self):
        if getattr(self, "_h", None) and self._h.value:
            lib().sgat_plan_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def device_bytes(self) -> int:
        b = ctypes.c_size_t()
        _check("sgat_plan_device_bytes", lib().sgat_plan_device_bytes(self._h, ctypes.byref(b)))
        return int(b.value)

    def upload(self, buf, stream=None):
        """Copy the plan into the caller's device buffer (a uint8 torch tensor)."""
        _check("sgat_plan_upload",
               lib().sgat_plan_upload(self._h, _ptr(buf), buf.numel() * buf.element_size(),
                                      _stream(stream)))
        self._dev = buf          # the plan reads it for as long as it is used

    def stats(self) -> dict:
        s = PlanStats()
        _check("sgat_plan_stats_get", lib().sgat_plan_stats_get(self._h, ctypes.byref(s)))
        return {name: int(getattr(s, name)) for name, _ in PlanStats._fields_}

    def export(self, array_id: int) -> np.ndarray:
        b = ctypes.c_size_t()
        _check("sgat_plan_array_bytes",
               lib().sgat_plan_array_bytes(self._h, array_id, ctypes.byref(b)))
        dt = ARRAY_DTYPES[array_id]
        out = np.empty(int(b.value) // dt.itemsize, dtype=dt)
        _check("sgat_plan_export",
               lib().sgat_plan_export(self._h, array_id, out.ctypes.data if out.size else None,
                                      int(b.value)))
        return out

    def workspace_bytes(self, op: int, heads: int, dim: int, dtype: int) -> int:
        b = ctypes.c_size_t()
        _check("sgat_workspace_bytes",
               lib().sgat_workspace_bytes(self._h, op, heads, dim, dtype, ctypes.byref(b)))
        return int(b.value)


# ---------------------------------------------------------------------------
# entry points (same names and argument order as the C ABI)
# ---------------------------------------------------------------------------

def gt_fwd(plan: Plan, rowptr, colidx, q, k, v, out, lse, ws, use_tiles=False, stream=None):
    import torch
    n, H, D = _shape(q)
    dev = _check_call(plan, rowptr, colidx, ws, q)
    for nm, t in (("q", q), ("k", k), ("v", v), ("out", out)):
        _expect(nm, t, q.shape, q.dtype, dev)
    _expect("lse", lse, (n, H), torch.float32, dev)
    _check("gt_fwd", lib().gt_fwd(
        plan.handle, plan.n, plan.nnz, _ptr(rowptr), _ptr(colidx), H, D, _dtype_code(q),
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
        _ptr(ws), _ws_bytes(ws), int(bool(use_tiles)), _stream(stream)))


def gt_fwd_noalloc(plan: Plan, rowptr, colidx, q, k, v, out, lse, use_tiles=False, stream=None):
    """gt_fwd with the library's static scratch instead of a workspace (for
    callers that cannot allocate; calls on one GPU must not overlap)."""
    import torch
    n, H, D = _shape(q)
    dev = _check_call(plan, rowptr, colidx, None, q)
    for nm, t in (("q", q), ("k", k), ("v", v), ("out", out)):
        _expect(nm, t, q.shape, q.dtype, dev)
    _expect("lse", lse, (n, H), torch.float32, dev)
    _check("gt_fwd_noalloc", lib().gt_fwd_noalloc(
        plan.handle, plan.n, plan.nnz, _ptr(rowptr), _ptr(colidx), H, D, _dtype_code(q),
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), int(bool(use_tiles)), _stream(stream)))


def gt_bwd(plan: Plan, rowptr, colidx, q, k, v, out, lse, dout, dq, dk, dv, ws,
           use_tiles=False, stream=None):
    import torch
    n, H, D = _shape(q)
    dev = _check_call(plan, rowptr, colidx, ws, q)
    for nm, t in (("q", q), ("k", k), ("v", v), ("out", out), ("dout", dout), ("dq", dq),
                  ("dk", dk), ("dv", dv)):
        _expect(nm, t, q.shape, q.dtype, dev)
    _expect("lse", lse, (n, H), torch.float32, dev)
    _check("gt_bwd", lib().gt_bwd(
        plan.handle, plan.n, plan.nnz, _ptr(rowptr), _ptr(colidx), H, D, _dtype_code(q),
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(dout),
        _ptr(dq), _ptr(dk), _ptr(dv), _ptr(ws), _ws_bytes(ws),
        int(bool(use_tiles)), _stream(stream)))


def gat_fwd(plan: Plan, rowptr, colidx, x_dst, x_nbr, a, negative_slope, out, lse, ws,
            stream=None):
    import torch
    n, H, D = _shape(x_dst)
    dev = _check_call(plan, rowptr, colidx, ws, x_dst, "x_dst")
    for nm, t in (("x_nbr", x_nbr), ("out", out)):
        _expect(nm, t, x_dst.shape, x_dst.dtype, dev)
    _expect("a", a, (H, D), torch.float32, dev)
    _expect("lse", lse, (n, H), torch.float32, dev)
    _check("gat_fwd", lib().gat_fwd(
        plan.handle, plan.n, plan.nnz, _ptr(rowptr), _ptr(colidx), H, D, _dtype_code(x_dst),
        _ptr(x_dst), _ptr(x_nbr), _ptr(a), float(negative_slope), _ptr(out), _ptr(lse),
        _ptr(ws), _ws_bytes(ws), _stream(stream)))


def gat_bwd(plan: Plan, rowptr, colidx, x_dst, x_nbr, a, negative_slope, out, lse, dout,
            dx_dst, dx_nbr, da, ws, stream=None):
    import torch
    n, H, D = _shape(x_dst)
    dev = _check_call(plan, rowptr, colidx, ws, x_dst, "x_dst")
    for nm, t in (("x_nbr", x_nbr), ("out", out), ("dout", dout), ("dx_dst", dx_dst),
                  ("dx_nbr", dx_nbr)):
        _expect(nm, t, x_dst.shape, x_dst.dtype, dev)
    _expect("a", a, (H, D), torch.float32, dev)
    _expect("da", da, (H, D), torch.float32, dev)
    _expect("lse", lse, (n, H), torch.float32, dev)
    _check("gat_bwd", lib().gat_bwd(
        plan.handle, plan.n, plan.nnz, _ptr(rowptr), _ptr(colidx), H, D, _dtype_code(x_dst),
        _ptr(x_dst), _ptr(x_nbr), _ptr(a), float(negative_slope), _ptr(out), _ptr(lse),
        _ptr(dout), _ptr(dx_dst), _ptr(dx_nbr), _ptr(da), _ptr(ws),
        _ws_bytes(ws), _stream(stream)))


def _shape2(t):
    if t.dim() != 2:
        raise ValueError("aggregation tensors are [N, F]")
    return t.shape


def reduce_fwd(plan: Plan, rowptr, colidx, x, op, out, arg, ws, stream=None):
    """op: REDUCE_MIN / REDUCE_MAX (or "min" / "max"); arg may be None."""
    import torch
    n, F = _shape2(x)
    dev = _check_call(plan, rowptr, colidx, ws, x, "x")
    _expect("out", out, x.shape, x.dtype, dev)
    if arg is not None:
        _expect("arg", arg, (n, F), torch.int32, dev)
    op = REDUCE_OPS.get(op, op)
    _check("reduce_fwd", lib().reduce_fwd(
        plan.handle, plan.n, plan.nnz, _ptr(rowptr), _ptr(colidx), F, _dtype_code(x), int(op),
        _ptr(x), _ptr(out), _ptr(arg), _ptr(ws), _ws_bytes(ws), _stream(stream)))


def reduce_bwd(plan: Plan, rowptr, colidx, arg, dout, dx, ws, stream=None):
    import torch
    n, F = _shape2(dout)
    dev = _check_call(plan, rowptr, colidx, ws, dout, "dout")
    _expect("arg", arg, (n, F), torch.int32, dev)
    _expect("dx", dx, dout.shape, dout.dtype, dev)
    _check("reduce_bwd", lib().reduce_bwd(
        plan.handle, plan.n, plan.nnz, _ptr(rowptr), _ptr(colidx), F, _dtype_code(dout),
        _ptr(arg), _ptr(dout), _ptr(dx), _ptr(ws), _ws_bytes(ws), _stream(stream)))


# ---------------------------------------------------------------------------
# trace
# ---------------------------------------------------------------------------

def trace_enable(on: bool = True):
    _check("sgat_trace_enable", lib().sgat_trace_enable(int(bool(on))))


def trace_only(name: str | None = None):
    """Trace only the kernels of this name (None: every kernel)."""
    _check("sgat_trace_only", lib().sgat_trace_only(name.encode() if name else None))


def trace_clear():
    _check("sgat_trace_clear", lib().sgat_trace_clear())


def trace_read() -> list:
    """[(kernel name, milliseconds)] of the traced launches (stream synced first)."""
    out = []
    name = ctypes.create_string_buffer(64)
    ms = ctypes.c_float()
    for i in range(lib().sgat_trace_count()):
        _check("sgat_trace_get", lib().sgat_trace_get(i, name, 64, ctypes.byref(ms)))
        out.append((name.value.decode(), float(ms.value)))
    return out


def probe_read(buf, sink, blocks: int = 2048, stream=None):
    """Stream the bytes of a device tensor (sgat_probe_read)."""
    _check("sgat_probe_read", lib().sgat_probe_read(
        _ptr(buf), buf.numel() * buf.element_size(), _ptr(sink), int(blocks), _stream(stream)))


def probe_gather(table, idx, sink, stream=None):
    """Gather rows of a 2-D device tensor at device int32 indices (sgat_probe_gather)."""
    row_bytes = table.shape[1] * table.element_size()
    _check("sgat_probe_gather", lib().sgat_probe_gather(
        _ptr(table), table.shape[0], row_bytes, _ptr(idx), idx.numel(), _ptr(sink),
        _stream(stream)))


# ---------------------------------------------------------------------------
# convenience: a graph resident on one device
# ---------------------------------------------------------------------------

class DeviceGraph:
    """A CSR graph with its plan uploaded to one device.

    Holds the device copies of rowptr/colidx, the plan and its device buffer,
    and hands out workspaces of the size the library asks for.
    """

    def __init__(self, rowptr, colidx, device="cuda", chunk: int = 0, tile_min_nnz: int = 0,
                 block_sparse: bool = False, locality: bool = False, edge_order: int = 0,
                 stream=None):
        import torch
        self.plan = Plan(rowptr, colidx, chunk=chunk, tile_min_nnz=tile_min_nnz,
                         block_sparse=block_sparse, locality=locality, edge_order=edge_order)
        self.n, self.nnz = self.plan.n, self.plan.nnz
        self.device = torch.device(device)
        self.rowptr = torch.from_numpy(np.ascontiguousarray(rowptr, dtype=np.int64)).to(self.device)
        self.colidx = torch.from_numpy(np.ascontiguousarray(colidx, dtype=np.int32)).to(self.device)
        self.plan_buf = torch.empty(self.plan.device_bytes(), dtype=torch.uint8, device=self.device)
        self.plan.upload(self.plan_buf, stream)
        self._ws = {}

    def workspace(self, op: int, heads: int, dim: int, dtype: int):
        import torch
        nb = self.plan.workspace_bytes(op, heads, dim, dtype)
        key = (op, heads, dim, dtype)
        ws = self._ws.get(key)
        if ws is None or ws.numel() < nb:
            ws = torch.empty(max(nb, 1), dtype=torch.uint8, device=self.device)
            self._ws[key] = ws
        return ws
