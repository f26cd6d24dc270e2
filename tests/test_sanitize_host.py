"""The C ABI's host code (validation, workspace carving, the host-side sampler grid) built with
AddressSanitizer and UndefinedBehaviorSanitizer and exercised on the CPU by
tests/sanitize/abi_host_checks.cpp: every call there fails validation or only queries sizes before any
device work, so no GPU is needed. Needs hipcc and the objects of the normal library build."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OBJ = os.path.join(ROOT, "flow_matching_diffusion_amd", "_build")
HIPCC = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")


def test_abi_host_code_under_asan_and_ubsan(tmp_path):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    objs = ["gemm.o", "attention.o", "elementwise.o", "backward.o", "probe.o"]
    if not all(os.path.exists(os.path.join(OBJ, o)) for o in objs):
        pytest.skip("library objects not built (run __graft_entry__.build() first)")
    r = subprocess.run(["bash", os.path.join(ROOT, "tests", "sanitize", "build_and_run.sh"), str(tmp_path)],
                       capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "OK: 0 failure(s)" in r.stdout
    assert "AddressSanitizer" not in out and "runtime error" not in out
