"""The host runtime (validation, grouping, chunk and split planning, workspace
sizing) under AddressSanitizer and UndefinedBehaviorSanitizer.

runtime.cpp is recompiled with the sanitizers on its host code only
(-Xarch_host) and linked with the regular kernel objects into a separate
library; tests/abi_sanitize_driver.c calls the host-only entry points on every
workload's shape list and on the documented rejections, with fake device
pointers.  Nothing touches a GPU, so this runs on the CPU."""

import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BUILD = os.path.join(ROOT, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def _run(cmd, **kw):
    res = subprocess.run(cmd, capture_output=True, text=True, **kw)
    if res.returncode != 0:
        raise AssertionError(f"{' '.join(cmd)}\nrc={res.returncode}\n{res.stdout[-4000:]}\n{res.stderr[-4000:]}")
    return res


def test_host_runtime_under_asan_and_ubsan(tmp_path):
    from muon_step_amd import build as b
    objs = [os.path.join(BUILD, src + ".o") for src in b.SOURCES if src != "runtime.cpp"]
    if not all(os.path.exists(o) for o in objs):
        pytest.fail("kernel objects are not built (run __graft_entry__.build())")
    rt = str(tmp_path / "runtime_san.o")
    _run([HIPCC, *b.COMMON, *SAN, "-c", os.path.join(b.CSRC, "runtime.cpp"), "-o", rt])
    lib = str(tmp_path / "libmuon_step_san.so")
    _run([HIPCC, "-shared", "-fPIC", f"--offload-arch={b.ARCH}", *SAN, rt, *objs, "-o", lib])
    exe = str(tmp_path / "driver")
    _run([HIPCC, *SAN, "-x", "c", "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
          os.path.join(ROOT, "tests", "abi_sanitize_driver.c"), "-x", "none", lib, "-o", exe,
          f"-Wl,-rpath,{tmp_path}"])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    res = _run([exe], env=env, timeout=300)
    assert "sanitized host checks: ok" in res.stdout
    assert "runtime error" not in res.stderr
