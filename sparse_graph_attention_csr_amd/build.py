"""Build libsgattn.so (HIP for gfx950) in-tree.

    python -m sparse_graph_attention_csr_amd.build [--sanitize]

Each source is compiled by hipcc into _build/, in parallel, then linked into
sparse_graph_attention_csr_amd/libsgattn.so. Packed fp32 VALU instructions are
disabled for all device code.

--sanitize builds _build/san/libsgattn_san.so instead, with the host code
(plan construction, CSR validation, the C ABI's checks) instrumented by
AddressSanitizer and UndefinedBehaviorSanitizer; the device code is built as
usual. Load it with SGAT_LIBRARY=<path> and clang's ASan runtime preloaded
(tests/run_sanitized.sh does both).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libsgattn.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["plan.cpp", "api.cpp", "launch_gt.hip", "launch_gat.hip", "launch_bs.hip",
           "launch_reduce.hip", "probe.hip"]

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++20", "-fPIC", "-Wall", "-Wno-unused-result",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


SAN_BUILD = os.path.join(BUILD, "san")
SAN_LIB = os.path.join(SAN_BUILD, "libsgattn_san.so")
# host-side instrumentation only: every sanitizer flag applies to the host pass
SAN_FLAGS = ["-g", "-Xarch_host", "-fno-omit-frame-pointer",
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined"]


def _compile(src: str, sanitize: bool = False) -> str:
    path = os.path.join(CSRC, src)
    obj = os.path.join(SAN_BUILD if sanitize else BUILD, src + ".o")
    cmd = [HIPCC, "-x", "hip", *FLAGS, *(SAN_FLAGS if sanitize else []), "-c", path, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (r.stderr or "").splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def build(jobs: int | None = None, sanitize: bool = False) -> str:
    os.makedirs(SAN_BUILD if sanitize else BUILD, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 4)
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, sanitize), SOURCES))
    lib = SAN_LIB if sanitize else LIB
    tmp = lib + ".tmp"
    link = SAN_FLAGS if sanitize else []
    subprocess.check_call([HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", *link, "-o", tmp,
                           *objs])
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(sanitize="--sanitize" in sys.argv[1:]))
