"""The library's host C++ code (layout builder, height tuning, reuse selection) under
sanitizers, on the CPU: `tests/host_sanitize.c` linked with the three host sources, built
once with AddressSanitizer + UndefinedBehaviorSanitizer and once with ThreadSanitizer (the
layout builder splits large matrices over worker threads). No HIP code is built or run."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mixed_precision_sparse_amd", "csrc")
HOST_SOURCES = ["mpcg_layout.cpp", "mpcg_reuse.cpp", "mpcg_tuning.cpp"]


def _build_and_run(tmp_path, flags, env_extra):
    if not shutil.which("gcc") or not shutil.which("g++"):
        pytest.skip("gcc/g++ not available")
    inc = os.path.join(ROOT, "include")
    objs = []
    drv = str(tmp_path / "driver.o")
    subprocess.run(["gcc", "-std=c99", "-O1", "-g", "-fno-omit-frame-pointer", *flags, f"-I{inc}", "-c",
                    os.path.join(ROOT, "tests", "host_sanitize.c"), "-o", drv], check=True)
    objs.append(drv)
    for src in HOST_SOURCES:
        obj = str(tmp_path / (src + ".o"))
        subprocess.run(["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", *flags, f"-I{inc}", "-c",
                        os.path.join(CSRC, src), "-o", obj], check=True)
        objs.append(obj)
    exe = str(tmp_path / "host_sanitize")
    subprocess.run(["g++", *flags, *objs, "-o", exe, "-lpthread", "-lm"], check=True)
    env = dict(os.environ, **env_extra)
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    return r


def test_host_code_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    r = _build_and_run(tmp_path, ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined"],
                       {"ASAN_OPTIONS": "detect_leaks=1:halt_on_error=1:verify_asan_link_order=0",
                        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"})
    assert r.returncode == 0 and "host_sanitize: ok" in r.stdout, (r.stdout[-3000:], r.stderr[-3000:])
    assert "runtime error" not in r.stderr and "ERROR: AddressSanitizer" not in r.stderr, r.stderr[-3000:]


def test_host_code_under_thread_sanitizer(tmp_path):
    r = _build_and_run(tmp_path, ["-fsanitize=thread"], {"TSAN_OPTIONS": "halt_on_error=1"})
    assert r.returncode == 0 and "host_sanitize: ok" in r.stdout, (r.stdout[-3000:], r.stderr[-3000:])
    assert "WARNING: ThreadSanitizer" not in r.stderr, r.stderr[-3000:]
