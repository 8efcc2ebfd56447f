"""The C-ABI checks again, against a host-side AddressSanitizer + UndefinedBehaviorSanitizer
build of the ABI file (api.cpp), CPU only.

The ABI file is recompiled with the sanitizers on its host code (device code untouched) and
linked with the other objects of the regular build into a scratch library; tests/test_abi.py
then runs in a child process that loads that library with the sanitizer runtime preloaded.
Any report (out-of-bounds access, use after free, undefined behaviour such as an
out-of-range enum load) aborts the child and fails this test.
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "block_verify_sv_amd")
BUILD = os.path.join(PKG, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/llvm/bin/clang++"


def _asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


@pytest.mark.slow
def test_abi_checks_under_host_sanitizers(tmp_path):
    rt = _asan_runtime()
    objs = [o for o in glob.glob(os.path.join(BUILD, "*.o"))
            if os.path.basename(o) not in ("api.o", "hbm_probe.o")]
    if rt is None or not os.path.exists(CLANG) or not objs:
        pytest.skip("needs the ROCm clang sanitizer runtime and a regular build's objects")
    api_o = str(tmp_path / "api_sanitized.o")
    lib = str(tmp_path / "libspecverify_sanitized.so")
    compile_cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
                   "-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc"),
                   "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                   "-Xarch_host", "-fno-omit-frame-pointer", "-Wno-unused-command-line-argument",
                   "-c", os.path.join(PKG, "csrc", "api.cpp"), "-o", api_o]
    r = subprocess.run(compile_cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    link_cmd = [CLANG, "-shared", "-fPIC", "-fsanitize=address,undefined", "-shared-libasan",
                "-o", lib, api_o] + objs + ["-L/opt/rocm/lib", "-lamdhip64",
                                            "-Wl,-rpath,/opt/rocm/lib"]
    r = subprocess.run(link_cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    child = ("import sys; sys.path.insert(0, %r); import block_verify_sv_amd as sv; "
             "sv.LIB_PATH = %r; import pytest; "
             "sys.exit(pytest.main(['-q', '-x', '-p', 'no:cacheprovider', %r]))"
             % (ROOT, lib, os.path.join(ROOT, "tests", "test_abi.py")))
    env = dict(os.environ, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-c", child], capture_output=True, text=True, env=env,
                       cwd=ROOT, timeout=600)
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert " passed" in r.stdout
