"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(no GPU needed): dg_canvas.hip is rebuilt with the sanitizers on its host
side only (-Xarch_host; the device code is unchanged), linked with the other
objects into a separate library, and tests/abi_host_check.cpp drives the
validation, schedule, accounting and NULL-handle paths against it."""
import os
import shutil
import subprocess

import pytest

from canvas_sampler_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
            "-Xarch_host", "-g"]


def _clangxx():
    for cand in ("/opt/rocm/lib/llvm/bin/clang++", shutil.which("amdclang++") or ""):
        if cand and os.path.exists(cand):
            return cand
    pytest.skip("no clang++ with sanitizer runtimes")


def test_host_abi_under_sanitizers(tmp_path):
    hipcc = build.hipcc()
    clangxx = _clangxx()
    objs = []
    for src in build.SOURCES:
        obj = str(tmp_path / src.replace(".hip", ".o"))
        prebuilt = os.path.join(ROOT, "_build", src.replace(".hip", ".o"))
        if src != "dg_canvas.hip" and os.path.exists(prebuilt):
            shutil.copy(prebuilt, obj)
        else:
            extra = HOST_SAN if src == "dg_canvas.hip" else []
            subprocess.run([hipcc] + build.flags() + extra + ["-c", os.path.join(build.CSRC, src), "-o", obj],
                           check=True, capture_output=True)
        objs.append(obj)
    lib = str(tmp_path / "libdgcanvas_san.so")
    subprocess.run([hipcc, "--offload-arch=" + build.ARCH, "-shared", "-fPIC"] + objs + ["-o", lib],
                   check=True, capture_output=True)
    exe = str(tmp_path / "abi_host_check")
    rocm_lib = "/opt/rocm/lib"
    subprocess.run([clangxx, "-std=c++17", "-g", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=undefined", "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "abi_host_check.cpp"), lib, "-L", rocm_lib, "-lamdhip64",
                    "-Wl,-rpath," + str(tmp_path) + ":" + rocm_lib, "-o", exe],
                   check=True, capture_output=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", HIP_VISIBLE_DEVICES="")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "host ABI checks passed" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr
