"""Fused sparse graph attention (Graph Transformer, GATv2) for AMD MI355X.

The compute lives in libsgattn.so (HIP for gfx950, C ABI in include/sgattn.h);
``binding`` is its ctypes binding and ``inputs`` the seeded synthetic
workloads. Names of the binding are re-exported lazily, so importing the
package (or ``inputs``) does not load the library.
"""
from importlib import import_module

_BINDING_NAMES = {
    "Plan", "DeviceGraph", "SgatError", "gt_fwd", "gt_bwd", "gat_fwd", "gat_bwd",
    "trace_enable", "trace_clear", "trace_read", "lib", "status_string",
    "F32", "BF16", "OP_GT_FWD", "OP_GT_BWD", "OP_GAT_FWD", "OP_GAT_BWD",
}


def __getattr__(name):
    if name in _BINDING_NAMES:
        return getattr(import_module(".binding", __name__), name)
    raise AttributeError(name)
