"""Host-only checks of the library's planner, argument checks and workspace
layouts (integer_only_dnn_amd/csrc/ie_plan.cpp), compiled with g++ under the
address and undefined-behaviour sanitizers together with tests/plan_check.cpp:
every plan the library would run writes only inside the workspace buffers
carved for it, forced plans that have no kernel or would split a group in a
direct epilogue are refused, and the convolution geometry is free of
undefined behaviour at the ends of its ranges.  No GPU is involved."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = [os.path.join(ROOT, "tests", "plan_check.cpp"),
       os.path.join(ROOT, "integer_only_dnn_amd", "csrc", "ie_plan.cpp")]


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    cxx = shutil.which(os.environ.get("CXX", "g++"))
    if cxx is None:
        pytest.skip("no host C++ compiler")
    exe = str(tmp_path_factory.mktemp("plan_check") / "plan_check")
    cmd = [cxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", *SRC, "-o", exe]
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert res.returncode == 0, res.stderr[-4000:]
    return exe


def test_plans_and_workspace_layouts_under_sanitizers(checker):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    res = subprocess.run([checker], capture_output=True, text=True, timeout=600, env=env)
    assert res.returncode == 0, (res.stdout + res.stderr)[-4000:]
    assert "plan_check:" in res.stdout
