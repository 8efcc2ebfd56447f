"""Build libspecverify.so in-tree with hipcc for gfx950.

    python -m block_verify_sv_amd.build          # compile every source, link the libraries

Objects go to ``block_verify_sv_amd/_build/``; the library to
``block_verify_sv_amd/libspecverify.so``.  The streaming-read probe the benchmark uses
for its bandwidth ceiling and the Philox probe the tests use to compare the device
generator's words with the oracle's are linked on their own into ``libsvprobe.so``
(measurement and test only; the verification library does not contain them).  Every
call recompiles.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libspecverify.so")
PROBE_LIB = os.path.join(PKG, "libsvprobe.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["api.cpp", "attention.hip", "accept_greedy.hip", "accept_sample.hip",
           "compress.hip", "kv_append.hip", "commit.hip", "lm_head.hip", "noalloc.hip",
           "accept_sample_tree.hip"]
PROBE_SOURCES = ["hbm_probe.hip", "philox_probe.hip"]

COMMON = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-I", os.path.join(ROOT, "include"), "-I", SRC,
    # packed fp32 arithmetic stays off: plain fp32 code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # leading scalar and pointer kernel arguments arrive preloaded in SGPRs, so a kernel's
    # first loads need no kernel-argument round trip (an aggregate argument ends the run)
    "-Xarch_device", "-mllvm=-amdgpu-kernarg-preload-count=16",
    "-Wno-unused-command-line-argument",
]


def _compile(src):
    obj = os.path.join(OUT, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [HIPCC] + COMMON + lang + ["-c", os.path.join(SRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, lib):
    tmp = lib + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    os.makedirs(OUT, exist_ok=True)
    srcs = SOURCES + PROBE_SOURCES
    with ThreadPoolExecutor(max_workers=min(len(srcs), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(_compile, srcs))
    _link(objs[:len(SOURCES)], LIB)
    _link(objs[len(SOURCES):], PROBE_LIB)
    if verbose:
        print(f"built {LIB} and {PROBE_LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
