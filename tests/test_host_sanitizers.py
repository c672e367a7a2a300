"""The host half of libsplitkv (argument checks, chunk costs, LPT, the split
planner, the per-XCD planner and the schedule image it lays out word by
word) built with
AddressSanitizer and UndefinedBehaviorSanitizer by the host compiler, linked
with the normally built device objects, and the CPU tests of the C ABI run
against it in a child process.  An out-of-bounds write into the schedule
image, a signed overflow or a misaligned access in the host code aborts the
child with a report.  No device call is made."""
import os
import subprocess
import sys

import pytest

from block_sparse_split_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_sparse_split_amd", "csrc")
HOST_SOURCES = ["host.cpp", "timing.cpp"]
DEVICE_OBJECTS = ["fwd.o", "merge.o", "bwd.o", "noalloc.o"]
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all"]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


def _runtime(name):
    path = subprocess.run(["g++", f"-print-file-name={name}"], capture_output=True,
                          text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def _sanitized_library(out):
    objs = []
    for src in HOST_SOURCES:
        obj = os.path.join(out, src.replace(".cpp", ".o"))
        _run(["g++", "-O1", "-g", "-std=c++17", "-fPIC", "-fno-omit-frame-pointer", *SAN,
              "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I", os.path.join(ROOT, "include"),
              "-I", CSRC, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    dev = [os.path.join(build.BUILD, o) for o in DEVICE_OBJECTS]
    if not all(os.path.exists(o) for o in dev):
        build.build()
    lib = os.path.join(out, "libsplitkv_san.so")
    _run(["g++", "-shared", *SAN, *objs, *dev, "-L/opt/rocm/lib", "-lamdhip64",
          "-Wl,-rpath,/opt/rocm/lib", "-o", lib])
    return lib


@pytest.mark.skipif(_runtime("libasan.so") is None, reason="no AddressSanitizer runtime")
def test_cpu_abi_tests_are_clean_under_asan_and_ubsan(tmp_path):
    lib = _sanitized_library(str(tmp_path))
    nm = _run(["nm", "-D", lib]).stdout
    assert "__asan_report" in nm and "__ubsan_handle" in nm   # really instrumented
    env = dict(os.environ)
    # the sanitizer runtime first, then the C++ runtime whose throw it wraps
    env["LD_PRELOAD"] = f"{_runtime('libasan.so')} {_runtime('libstdc++.so.6') or ''}".strip()
    env["SKV_LIBRARY"] = lib
    logs = tmp_path / "logs"
    logs.mkdir()
    log = str(logs / "san")
    env["ASAN_OPTIONS"] = f"detect_leaks=0:halt_on_error=1:log_path={log}"
    env["UBSAN_OPTIONS"] = f"print_stacktrace=1:halt_on_error=1:log_path={log}"
    tests = [os.path.join(ROOT, "tests", f) for f in
             ("test_abi_cpu.py", "test_plan_split_cpu.py", "test_xcd_plan_cpu.py",
              "test_bench_host.py")]
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        "-m", "not gpu", *tests], capture_output=True, text=True, env=env,
                       cwd=ROOT, timeout=600)
    reports = [open(os.path.join(logs, f)).read() for f in os.listdir(logs)]
    assert r.returncode == 0 and not reports, (r.stdout[-3000:], r.stderr[-3000:], reports)
    assert " passed" in r.stdout
