"""The C ABI without a GPU: the library loads, exports every function the
header declares, and rejects invalid arguments with the documented status
before any HIP call (fake non-null device pointers are never dereferenced)."""
import ctypes
import os
import re

import numpy as np
import pytest

from sparse_graph_attention_csr_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    src = open(os.path.join(ROOT, "include", "sgattn.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(\w+)\s*\(", src, flags=re.M)
    return sorted(set(names))


def test_library_exports_every_declared_function():
    names = header_functions()
    assert len(names) >= 17
    L = B.lib()
    missing = [n for n in names if not hasattr(L, n)]
    assert not missing, missing
    assert set(names) == set(B._SIGS), "binding signatures out of sync with the header"


def test_status_strings():
    for st in range(10):
        assert B.status_string(st) != "unknown status"
    assert B.status_string(99) == "unknown status"


FAKE = 1 << 20   # aligned, non-null, never dereferenced


@pytest.fixture()
def plan():
    rp = np.array([0, 2, 3, 3, 5], dtype=np.int64)
    ci = np.array([0, 1, 2, 1, 3], dtype=np.int32)
    return B.Plan(rp, ci, chunk=1)


def call_gt_fwd(plan, n=None, nnz=None, H=2, D=32, dt=0, q=FAKE, lse=FAKE, ws=FAKE, wsb=1 << 30,
                tiles=0):
    return B.lib().gt_fwd(plan.handle if plan is not None else None,
                          plan.n if n is None else n, plan.nnz if nnz is None else nnz,
                          FAKE, FAKE, H, D, dt, q, FAKE, FAKE, FAKE, lse, ws, wsb, tiles, None)


def test_gt_fwd_argument_checks(plan):
    L = B.lib()
    assert L.gt_fwd(None, 4, 5, FAKE, FAKE, 2, 32, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, 0,
                    None) == 1
    assert call_gt_fwd(plan, H=0) == 1
    assert call_gt_fwd(plan, H=17) == 1
    assert call_gt_fwd(plan, D=48) == 1
    assert call_gt_fwd(plan, dt=2) == 1
    assert call_gt_fwd(plan, n=5) == 4
    assert call_gt_fwd(plan, nnz=4) == 4
    assert call_gt_fwd(plan) == 6            # not uploaded


def test_gt_fwd_noalloc_argument_checks(plan):
    """The static-scratch variant checks its arguments like gt_fwd, before it
    looks up the scratch or launches anything."""
    L = B.lib()

    def call(p=plan, H=2, D=32, dt=0, lse=FAKE, tiles=0):
        return L.gt_fwd_noalloc(p.handle if p is not None else None, plan.n, plan.nnz,
                                FAKE, FAKE, H, D, dt, FAKE, FAKE, FAKE, FAKE, lse, tiles, None)
    assert call(p=None) == 1
    assert call(H=0) == 1
    assert call(D=48) == 1
    assert call(dt=2) == 1
    assert call() == 6                       # plan not uploaded
    assert B.NOALLOC_SCRATCH_BYTES == 32 << 20
    hdr = open(os.path.join(ROOT, "include", "sgattn.h")).read()
    assert "#define SGAT_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)" in hdr


def test_workspace_bytes(plan):
    s = plan.stats()
    assert s["row_splits"] == 2 and s["row_slots"] == 4
    for op in range(4):
        for dt in (0, 1):
            nb = plan.workspace_bytes(op, 2, 32, dt)
            assert nb % 256 == 0
    # forward: partial accumulators and (max, sum) per slot, each region 256-aligned
    HD = 2 * 32
    fwd = plan.workspace_bytes(B.OP_GT_FWD, 2, 32, 1)
    assert fwd == (-(-4 * HD * 4 // 256) * 256) + (-(-4 * 2 * 8 // 256) * 256)
    with pytest.raises(B.SgatError):
        plan.workspace_bytes(7, 2, 32, 0)
    with pytest.raises(B.SgatError):
        plan.workspace_bytes(0, 2, 40, 0)


def test_upload_checks(plan):
    L = B.lib()
    nb = plan.device_bytes()
    assert nb > 0 and nb % 256 == 0
    assert L.sgat_plan_upload(plan.handle, None, nb, None) == 1
    assert L.sgat_plan_upload(plan.handle, FAKE, nb - 1, None) == 3
    assert L.sgat_plan_upload(plan.handle, FAKE + 8, nb, None) == 1


def test_export_checks(plan):
    L = B.lib()
    b = ctypes.c_size_t()
    assert L.sgat_plan_array_bytes(plan.handle, 22, ctypes.byref(b)) == 1
    assert L.sgat_plan_array_bytes(plan.handle, B.ARR_ROW_ITEMS, ctypes.byref(b)) == 0
    assert b.value == plan.stats()["row_items"] * 24
    buf = ctypes.create_string_buffer(b.value)
    assert L.sgat_plan_export(plan.handle, B.ARR_ROW_ITEMS, buf, b.value - 1) == 3


def test_other_entry_points_check_arguments(plan):
    L = B.lib()
    n, nnz = plan.n, plan.nnz
    args_bwd = [FAKE] * 9
    assert L.gt_bwd(plan.handle, n, nnz, FAKE, FAKE, 2, 64, 1, *args_bwd, FAKE, 1 << 30, 0,
                    None) == 6
    assert L.gt_bwd(plan.handle, n + 1, nnz, FAKE, FAKE, 2, 64, 1, *args_bwd, FAKE, 1 << 30, 0,
                    None) == 4
    assert L.gat_fwd(plan.handle, n, nnz, FAKE, FAKE, 2, 64, 1, FAKE, FAKE, FAKE, 0.2, FAKE, FAKE,
                     FAKE, 1 << 30, None) == 6
    assert L.gat_fwd(plan.handle, n, nnz, FAKE, FAKE, 2, 64, 3, FAKE, FAKE, FAKE, 0.2, FAKE, FAKE,
                     FAKE, 1 << 30, None) == 1
    assert L.gat_bwd(plan.handle, n, nnz, FAKE, FAKE, 2, 64, 1, FAKE, FAKE, FAKE, 0.2, FAKE, FAKE,
                     FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, None) == 6
    assert L.gat_bwd(None, n, nnz, FAKE, FAKE, 2, 64, 1, FAKE, FAKE, FAKE, 0.2, FAKE, FAKE,
                     FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, None) == 1


def test_plan_create_null_out():
    rp = np.array([0, 0], dtype=np.int64)
    assert B.lib().sgat_plan_create(1, 0, rp.ctypes.data, None, None, None) == 1


def test_trace_api_without_launches():
    B.trace_enable(True)
    B.trace_clear()
    assert B.trace_read() == []
    B.trace_enable(False)


def test_reduce_argument_checks(plan):
    L = B.lib()
    n, nnz = plan.n, plan.nnz

    def fwd(F=512, dt=1, op=0, h=plan.handle, n_=n, arg=FAKE, x=FAKE):
        return L.reduce_fwd(h, n_, nnz, FAKE, FAKE, F, dt, op, x, FAKE, arg, FAKE, 1 << 30, None)

    assert fwd(h=None) == 1
    assert fwd(F=0) == 1
    assert fwd(F=12) == 1                 # bf16 rows must be whole 16-byte fragments
    assert fwd(F=12, dt=0) == 6           # fp32: multiple of 4 is fine (then: not uploaded)
    assert fwd(F=4096) == 1               # above the maximum
    assert fwd(dt=2) == 1
    assert fwd(n_=n + 1) == 4
    assert fwd() == 6                     # not uploaded
    assert L.reduce_bwd(plan.handle, n, nnz, FAKE, FAKE, 64, 0, FAKE, FAKE, FAKE, FAKE, 1 << 30,
                        None) == 6
    assert L.reduce_bwd(plan.handle, n, nnz, FAKE, FAKE, 66, 0, FAKE, FAKE, FAKE, FAKE, 1 << 30,
                        None) == 1


def test_reduce_workspace_bytes(plan):
    s = plan.stats()
    F = 512
    fwd = plan.workspace_bytes(B.OP_REDUCE_FWD, 1, F, B.BF16)
    assert fwd == 2 * (-(-s["row_slots"] * F * 4 // 256) * 256)
    def up(x):
        return -(-x // 256) * 256

    for dt, eb in ((B.F32, 8), (B.BF16, 4)):
        bwd = plan.workspace_bytes(B.OP_REDUCE_BWD, 1, F, dt)
        assert bwd == up(s["col_slots"] * F * 4) + up(s["nnz"] * 4) + up(s["n"] * F * eb)
    with pytest.raises(B.SgatError):
        plan.workspace_bytes(B.OP_REDUCE_FWD, 2, F, B.BF16)      # H must be 1
    with pytest.raises(B.SgatError):
        plan.workspace_bytes(B.OP_REDUCE_FWD, 1, 4100, B.F32)


def test_plan_rejects_nnz_beyond_int32():
    """Edge positions are int32: nnz >= 2^31 is refused before any array is read."""
    rp = np.array([0, 1 << 31], dtype=np.int64)
    ci = np.zeros(1, dtype=np.int32)
    out = ctypes.c_void_p()
    assert B.lib().sgat_plan_create(1, 1 << 31, rp.ctypes.data, ci.ctypes.data, None,
                                    ctypes.byref(out)) == 1
    assert not out.value


def test_binding_refuses_host_tensors_before_any_call(plan):
    """The binding checks tensor arguments itself (the ABI sees bare pointers):
    host tensors never reach the library."""
    import torch
    n, H, D = plan.n, 2, 32
    q = torch.zeros(n, H, D)
    lse = torch.zeros(n, H)
    rp = torch.zeros(n + 1, dtype=torch.int64)
    ci = torch.zeros(plan.nnz, dtype=torch.int32)
    with pytest.raises(ValueError, match="GPU"):
        B.gt_fwd(plan, rp, ci, q, q, q, q.clone(), lse, None)
    with pytest.raises(ValueError, match="GPU"):
        B.reduce_fwd(plan, rp, ci, torch.zeros(n, 64), "min", torch.zeros(n, 64), None, None)
    with pytest.raises(ValueError, match="rows"):
        B.gt_fwd(plan, rp, ci, torch.zeros(n + 1, H, D), q, q, q, lse, None)


def test_missing_library_raises_without_fallback(tmp_path):
    """With no built library every entry point raises: there is no CPU path.
    Run in a child interpreter whose binding points at an empty directory."""
    import subprocess
    import sys
    code = (
        "import sparse_graph_attention_csr_amd.binding as B\n"
        f"B._LIB_PATH = {str(tmp_path / 'libsgattn.so')!r}\n"
        "import numpy as np\n"
        "for call in (lambda: B.lib(), lambda: B.Plan(np.array([0, 1]), np.array([0], np.int32)),\n"
        "             lambda: B.gt_fwd(None, None, None, None, None, None, None, None, None)):\n"
        "    try:\n"
        "        call()\n"
        "    except (RuntimeError, ValueError, AttributeError, TypeError):\n"
        "        pass\n"
        "    else:\n"
        "        raise SystemExit('a call succeeded without the library')\n"
        "try:\n"
        "    B.lib()\n"
        "except RuntimeError as e:\n"
        "    assert 'no fallback' in str(e)\n"
        "    print('raised')\n")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, "-c", code], cwd=root, capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0, r.stderr[-2000:]
    assert r.stdout.strip().endswith("raised")
