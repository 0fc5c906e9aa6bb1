"""Compile the HIP library libfp4w4a16.so for gfx950, in place (hipcc; no GPU needed), and the
benchmark's measurement probes, libfp4probe.so (a separate library outside the C ABI)."""
from __future__ import annotations

import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libfp4w4a16.so")
PROBE_LIB = os.path.join(HERE, "libfp4probe.so")
PROBE_SOURCES = ["probe.hip"]
BUILD_DIR = os.path.join(HERE, "_build")
SOURCES = ["api.hip", "layout.hip", "gemv.hip", "gemm.hip", "quantize.hip"]
ARCH = os.environ.get("FP4_OFFLOAD_ARCH", "gfx950")

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
    # no packed FP32 instructions anywhere in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # the GEMV and mid-M kernels take their leading 8 arguments (at most 12 dwords) in preloaded
    # scalar registers, so that a wave's first loads do not wait on the kernel-argument memory
    "-mllvm", "-amdgpu-kernarg-preload-count=8",
    "-Wno-unused-command-line-argument",
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, src + ".o")
    cmd = ["hipcc", "-c", os.path.join(CSRC, src), "-o", obj] + FLAGS
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def _link(objs: list[str], lib: str) -> None:
    tmp = lib + f".tmp{os.getpid()}"
    r = subprocess.run(["hipcc", "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs,
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = SOURCES + PROBE_SOURCES
    with ThreadPoolExecutor(max_workers=len(srcs)) as ex:
        objs = dict(zip(srcs, ex.map(_compile, srcs)))
    _link([objs[s] for s in SOURCES], LIB)
    _link([objs[s] for s in PROBE_SOURCES], PROBE_LIB)
    if verbose:
        print(LIB)
        print(PROBE_LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
