"""The host side of the C ABI (validation, launch planning, schedule, layout
maps: ringattn_abi.cpp) built with g++ under AddressSanitizer and
UndefinedBehaviorSanitizer, with stand-in launchers and no GPU code, then
driven by the host tests of the library (tests/test_host_abi.py) and by
successful calls of every entry point at the full workload shapes
(tests/host_sanitize/stubbed_launches.py), in a subprocess with the sanitizer
runtime preloaded.  Any report fails the test (CPU only)."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "exact_long_context_amd", "csrc")
HERE = os.path.join(ROOT, "tests", "host_sanitize")


def _gxx():
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not found")
    return gxx


def test_host_abi_under_asan_and_ubsan(tmp_path):
    gxx = _gxx()
    asan = subprocess.run([gxx, "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(asan) or not os.path.exists(asan):
        pytest.skip("libasan not available")
    # a copy of the tree the host tests need, with the sanitized build in place of the library
    for d in ("oracle", "synthetic", "include"):
        shutil.copytree(os.path.join(ROOT, d), tmp_path / d, ignore=shutil.ignore_patterns("__pycache__"))
    pkg = tmp_path / "exact_long_context_amd"
    pkg.mkdir()
    for f in ("__init__.py", "ringattn.py"):
        shutil.copy(os.path.join(ROOT, "exact_long_context_amd", f), pkg / f)
    tests = tmp_path / "tests"
    tests.mkdir()
    for f in ("__init__.py", "conftest.py", "test_host_abi.py"):
        shutil.copy(os.path.join(ROOT, "tests", f), tests / f)
    shutil.copy(os.path.join(HERE, "stubbed_launches.py"), tests / "stubbed_launches.py")
    shutil.copy(os.path.join(ROOT, "pytest.ini"), tmp_path / "pytest.ini")
    lib = pkg / "libringattn.so"
    cmd = [gxx, "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I", os.path.join(ROOT, "include"),
           "-I", CSRC, "-Wall", "-Wextra", "-Werror", "-shared", "-fPIC", "-g", "-O1", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           os.path.join(CSRC, "ringattn_abi.cpp"), os.path.join(HERE, "launch_stubs.cpp"), "-o", str(lib)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    env = dict(os.environ)
    env["LD_PRELOAD"] = asan + (":" + env["LD_PRELOAD"] if env.get("LD_PRELOAD") else "")
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["PYTHONDONTWRITEBYTECODE"] = "1"
    run = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "tests/test_host_abi.py",
                          "tests/stubbed_launches.py"], cwd=tmp_path, env=env, capture_output=True, text=True,
                         timeout=600)
    out = run.stdout + run.stderr
    print(out[-3000:])
    assert run.returncode == 0, out[-6000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out
    assert " passed" in out and " skipped" not in out
