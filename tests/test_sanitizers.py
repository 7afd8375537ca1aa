"""The CPU-side C and C++ of the repository under AddressSanitizer and
UndefinedBehaviorSanitizer (host code only; nothing here runs on a GPU):

* the oracle (oracle/lact_oracle.c) and the input generator (synth/synth.c), driven by
  tests/sanitize/oracle_driver.c through every entry point, multi-threaded attention
  included;
* the host planner (compressed_kv_causal_amd/csrc/plan.cpp), driven by
  tests/sanitize/plan_driver.cpp over 1000-step schedules of six configurations;
* the plain C client of the library's header (tests/c_client/plan_client.c), linked
  against the built liblact.so.

Each program is built in _build/sanitize with -fsanitize=address,undefined and
-fno-sanitize-recover=all, so any invalid access, leak (oracle and planner) or undefined
operation ends it with a non-zero status.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = os.path.join(ROOT, "_build", "sanitize")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
       "-g", "-O1"]


def _build_and_run(cmd, exe, env_extra=None, timeout=300):
    os.makedirs(OUT, exist_ok=True)
    r = subprocess.run(cmd + ["-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, f"build failed:\n{r.stderr}"
    env = dict(os.environ)
    env.update(env_extra or {})
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=timeout)
    assert r.returncode == 0, f"{os.path.basename(exe)} exited {r.returncode}:\n{r.stderr[-4000:]}"
    assert "runtime error" not in r.stderr and "ERROR: AddressSanitizer" not in r.stderr, r.stderr


def _tool(name):
    t = shutil.which(name)
    if t is None:
        pytest.skip(f"{name} not available")
    return t


def test_oracle_and_generator_under_sanitizers():
    gcc = _tool("gcc")
    _build_and_run([gcc, "-std=c11", *SAN, "-I", os.path.join(ROOT, "oracle"),
                    os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c"),
                    os.path.join(ROOT, "oracle", "lact_oracle.c"),
                    os.path.join(ROOT, "synth", "synth.c"), "-lm", "-lpthread"],
                   os.path.join(OUT, "oracle_driver"))


def test_planner_under_sanitizers():
    gxx = _tool("g++")
    _build_and_run([gxx, "-std=c++17", *SAN, "-I", os.path.join(ROOT, "include"),
                    "-I", os.path.join(ROOT, "compressed_kv_causal_amd", "csrc"),
                    os.path.join(ROOT, "tests", "sanitize", "plan_driver.cpp"),
                    os.path.join(ROOT, "compressed_kv_causal_amd", "csrc", "plan.cpp")],
                   os.path.join(OUT, "plan_driver"))


def test_c_client_under_sanitizers():
    gcc = _tool("gcc")
    lib_dir = os.path.join(ROOT, "compressed_kv_causal_amd")
    if not os.path.exists(os.path.join(lib_dir, "liblact.so")):
        pytest.skip("liblact.so is not built")
    # the client is instrumented; the library and the HIP runtime it loads are not, and the
    # runtime keeps allocations until exit, so leak reports are off for this one
    _build_and_run([gcc, "-std=c99", *SAN, "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "c_client", "plan_client.c"),
                    "-L", lib_dir, "-llact", "-Wl,-rpath," + lib_dir],
                   os.path.join(OUT, "plan_client"), env_extra={"ASAN_OPTIONS": "detect_leaks=0"})
