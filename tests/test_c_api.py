"""The C ABI used from a plain C99 program (tests/c/sgattn_c_api.c): no C++,
no torch, device memory from hipMalloc. On the CPU it checks the host-only
calls (plan, statistics, export, workspace sizes, argument errors); on the GPU
it also runs gt_fwd, gt_bwd, reduce_fwd and reduce_bwd and compares them with
the fp64 oracle linked into the program."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "c", "sgattn_c_api.c")
BIN = os.path.join(ROOT, "tests", "c", "sgattn_c_api")
LIB = os.path.join(ROOT, "sparse_graph_attention_csr_amd", "libsgattn.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build_c_program(force: bool = False) -> str:
    """gcc, C99, against include/sgattn.h and libsgattn.so (plus the oracle)."""
    deps = [SRC, os.path.join(ROOT, "oracle", "oracle.c"), os.path.join(ROOT, "include", "sgattn.h"),
            LIB]
    if not force and os.path.exists(BIN) and all(os.path.getmtime(BIN) >= os.path.getmtime(d)
                                                 for d in deps if os.path.exists(d)):
        return BIN
    cmd = ["gcc", "-std=c99", "-O2", "-Wall", "-fopenmp", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"),
           SRC, os.path.join(ROOT, "oracle", "oracle.c"),
           "-L", os.path.dirname(LIB), "-lsgattn", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           "-lm", "-Wl,-rpath,$ORIGIN/../../sparse_graph_attention_csr_amd",
           "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-o", BIN]
    subprocess.check_call(cmd)
    return BIN


def run(*args):
    r = subprocess.run([build_c_program(), *args], capture_output=True, text=True, timeout=120)
    return r.returncode, r.stdout + r.stderr


def test_c_program_host_calls():
    rc, out = run()
    assert rc == 0, out


@pytest.mark.gpu
def test_c_program_on_gpu():
    rc, out = run("gpu")
    assert rc == 0, out
    assert "gpu: 0 failure(s)" in out
