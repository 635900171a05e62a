"""The host library under ThreadSanitizer, and under AddressSanitizer with
UndefinedBehaviorSanitizer (CPU only, on the stand-in device).

The stress program tests/sanitize/driver.cpp (eight threads tuning shared and
private keys with the results file written through, saving, loading,
toggling options) is linked against the library's host sources built with
the sanitizer; the kernels' objects come from the normal build (their
device code never runs here).  A race, a memory error or undefined
behaviour fails the run, and so does any check inside that program.
"""
import os
import subprocess

import pytest

from gemm_autotuning_amd import build as b

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLANG = os.path.join(b.ROCM, "llvm", "bin", "clang++")
SAN = {
    "thread": ["-fsanitize=thread"],
    "address": ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined"],
}


def build_driver(kind, tmp):
    out = os.path.join(b.BUILD, "san_" + kind)
    os.makedirs(out, exist_ok=True)
    flags = [f for f in b.HOST_FLAGS if f != "-O2"] + ["-O1", "-g", "-fno-omit-frame-pointer"] + SAN[kind]
    objs = []
    jobs = []
    for src in [os.path.join(b.CSRC, n) for n in b.HOST_SOURCES] + [os.path.join(ROOT, "tests", "sanitize",
                                                                               "driver.cpp")]:
        obj = os.path.join(out, os.path.basename(src) + ".o")
        objs.append(obj)
        jobs.append(subprocess.Popen([CLANG] + flags + ["-I", os.path.join(ROOT, "include"), "-c", src, "-o", obj],
                                     stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True))
    for j in jobs:
        log, _ = j.communicate()
        assert j.returncode == 0, log
    kernels = b.kernel_objects()
    assert all(os.path.exists(k) for k in kernels), "the normal build has not run"
    exe = os.path.join(out, "driver")
    r = subprocess.run([CLANG] + SAN[kind] + ["-o", exe] + objs + kernels +
                       ["-L" + os.path.join(b.ROCM, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(b.ROCM, "lib"),
                        "-lpthread"], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    return exe


@pytest.mark.parametrize("kind", sorted(SAN))
def test_host_library_under_sanitizer(kind, tmp_path):
    exe = build_driver(kind, tmp_path)
    env = dict(os.environ)
    env["TSAN_OPTIONS"] = "halt_on_error=1:second_deadlock_stack=1"
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env.pop("LD_PRELOAD", None) if env.get("LD_PRELOAD", "").find("san") >= 0 else None
    r = subprocess.run([exe, str(tmp_path / "results.csv")], capture_output=True, text=True, timeout=600, env=env)
    assert r.returncode == 0, (r.stdout + r.stderr)[-6000:]
    assert "sanitize driver ok" in r.stdout
    assert "WARNING: ThreadSanitizer" not in r.stderr and "ERROR: AddressSanitizer" not in r.stderr
    assert "runtime error" not in r.stderr
