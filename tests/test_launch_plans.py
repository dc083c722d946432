"""The launch plans and workgroup-to-tile mappings of the kernels (optimizer_step_weight_amd/csrc/
forge_plan.h), checked on the host: tests/host_plan/plan_check.cpp compiles that header with the
host compiler and checks, for the workloads' shapes and many others, token counts (below and
above the wide-tile threshold, ragged), CU counts and input types, for the fused step and the
GEMM, that every 128 x 128 block of W is covered by exactly one workgroup and no tile leaves W.
tests/host_plan/queue_check.cpp does the same for the work queues of the one-launch backward step,
running the kernel's claim protocol under random interleavings.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def _build_and_run(tmp_path, name):
    if not shutil.which("g++"):
        pytest.skip("no host compiler")
    exe = tmp_path / name
    cmd = ["g++", "-std=c++17", "-O1", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__", "-I",
           os.path.join(ROOT, "optimizer_step_weight_amd", "csrc"), "-I", os.path.join(ROOT, "include"), "-I",
           os.path.join(ROCM, "include"), os.path.join(ROOT, "tests", "host_plan", name + ".cpp"), "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "0 failures" in r.stdout
    return r.stdout


def test_backward_work_queues_claim_every_item_once_and_dgrad_first(tmp_path):
    out = _build_and_run(tmp_path, "queue_check")
    print(out)


def test_every_element_is_covered_exactly_once(tmp_path):
    _build_and_run(tmp_path, "plan_check")
