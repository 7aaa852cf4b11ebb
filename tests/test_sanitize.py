"""The planner and the C ABI layer under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only).

A host-only build of planner.cpp and pod_api.cpp (kernel launchers replaced by
stubs that fail, see sanitize/launch_stubs.cpp) is compiled with g++ and the
planner and ABI tests run against it in a child process with the sanitizer
runtimes preloaded. A canary first checks that the sanitizer is live: a plan
written into an image buffer smaller than the capacity it claims must be
reported as a heap overflow."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "serving_attention_amd", "csrc")
OUT = os.path.join(ROOT, "_build", "san")
LIB = os.path.join(OUT, "libpod_attn_san.so")
ROCM = "/opt/rocm"


def _runtime(name):
    return subprocess.run(["g++", "-print-file-name=" + name], capture_output=True, text=True).stdout.strip()


@pytest.fixture(scope="module")
def san_env():
    if not os.path.exists(os.path.join(ROCM, "include", "hip", "hip_runtime.h")):
        pytest.skip("HIP headers not installed")
    os.makedirs(OUT, exist_ok=True)
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fPIC", "-shared", "-D__HIP_PLATFORM_AMD__",
           "-I" + os.path.join(ROCM, "include"), "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
           os.path.join(CSRC, "planner.cpp"), os.path.join(CSRC, "pod_api.cpp"),
           os.path.join(ROOT, "tests", "sanitize", "launch_stubs.cpp"),
           "-L" + os.path.join(ROCM, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(ROCM, "lib"),
           "-o", LIB]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    env = dict(os.environ)
    env["LD_PRELOAD"] = _runtime("libasan.so") + ":" + _runtime("libubsan.so")
    # CPython and torch keep memory until exit by design: leaks are not checked
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["POD_ATTN_LIB"] = LIB
    return env


CANARY = r"""
import ctypes, sys
import numpy as np
sys.path.insert(0, {root!r}); sys.path.insert(0, {tests!r})
from serving_attention_amd import _lib
from plan_helpers import plan_desc
assert _lib.LIB_PATH == {lib!r}
desc, keep = plan_desc(prefill=dict(qo_lens=[300], kv_lens=[700]), hqo=8, hkv=2)
lib = _lib.load()
info = _lib.PodPlanInfo()
lib.pod_plan_compute(ctypes.byref(desc), None, 0, ctypes.byref(info))
img = np.zeros(info.image_ints - 8, dtype=np.int32)    # the plan's last words fall past the end
lib.pod_plan_compute(ctypes.byref(desc), img.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                     info.image_ints, None)
print("canary not caught")
"""


def test_sanitizer_catches_an_overflow(san_env):
    code = CANARY.format(root=ROOT, tests=os.path.join(ROOT, "tests"), lib=LIB)
    res = subprocess.run([sys.executable, "-c", code], env=san_env, capture_output=True, text=True,
                         timeout=300)
    assert res.returncode != 0 and "heap-buffer-overflow" in res.stderr, res.stdout + res.stderr[-2000:]


def test_planner_and_abi_tests_are_clean_under_sanitizers(san_env):
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                          os.path.join(ROOT, "tests", "test_planner.py"),
                          os.path.join(ROOT, "tests", "test_abi.py")],
                         env=san_env, capture_output=True, text=True, timeout=900, cwd=ROOT)
    out = res.stdout + res.stderr
    assert res.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert " passed" in res.stdout
