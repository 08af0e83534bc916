"""Build libqmm.so (every HIP source, gfx950 only) in-tree.

    python -m quantized_matmul_qgemv_amd.build

Objects go to quantized_matmul_qgemv_amd/_build/, the library to
quantized_matmul_qgemv_amd/libqmm.so.  Each call recompiles everything.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libqmm.so")

SOURCES = ("qmm_api.hip", "qgemv.hip", "qgemm.hip", "qgemm_batched.hip", "moe.hip", "quant.hip")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 vector ops (v_pk_*_f32) stay disabled on this target
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *CFLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = min(len(SOURCES), max(1, min(8, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    shutil.move(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    build_dispatch_cost(verbose)
    build_stream_probe(verbose)
    return LIB


# Host dispatch-cost harness (dispatch_cost.hip): a C++ program linked
# against libqmm.so, run by bench.py.
DISPATCH_SRC = os.path.join(PKG, "dispatch_cost.hip")
DISPATCH_BIN = os.path.join(PKG, "qmm_dispatch_cost")


def build_dispatch_cost(verbose: bool = False) -> str:
    cmd = [HIPCC, *CFLAGS, "-O2", DISPATCH_SRC, f"-L{PKG}", "-lqmm", "-Wl,-rpath,$ORIGIN",
           "-o", DISPATCH_BIN]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on dispatch_cost.hip:\n{' '.join(cmd)}\n{r.stderr}")
    if verbose:
        print(f"built {DISPATCH_BIN}")
    return DISPATCH_BIN


# Streaming-rate harness (stream_probe.hip): a stand-alone program (no
# library code) that bench.py runs for the read-only rate of the GPU.
STREAM_SRC = os.path.join(PKG, "stream_probe.hip")
STREAM_BIN = os.path.join(PKG, "qmm_stream_probe")


def build_stream_probe(verbose: bool = False) -> str:
    cmd = [HIPCC, *CFLAGS, "-O2", STREAM_SRC, "-o", STREAM_BIN]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on stream_probe.hip:\n{' '.join(cmd)}\n{r.stderr}")
    if verbose:
        print(f"built {STREAM_BIN}")
    return STREAM_BIN


# Host-sanitizer build (AddressSanitizer + UndefinedBehaviorSanitizer on the
# host code only; the device code is built as usual).  Used by the CPU tests,
# which load it into a Python whose ASan runtime is preloaded.
SAN_BUILD = os.path.join(PKG, "_build_hostsan")
SAN_LIB = os.path.join(SAN_BUILD, "libqmm_hostsan.so")
SAN_FLAGS = [
    "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
    "-Xarch_host", "-g",
]


def asan_runtime() -> str:
    """The clang AddressSanitizer runtime that the sanitized build links against."""
    r = subprocess.run([os.path.join(os.path.dirname(HIPCC), "..", "llvm", "bin", "clang"),
                        "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("clang's libclang_rt.asan-x86_64.so was not found")
    return path


def build_host_sanitized(verbose: bool = False) -> str:
    """Build libqmm_hostsan.so (rebuilt only when a source or flag changed)."""
    import hashlib
    h = hashlib.sha256(" ".join(CFLAGS + SAN_FLAGS).encode())
    for d in (CSRC, INCLUDE):
        for f in sorted(os.listdir(d)):
            with open(os.path.join(d, f), "rb") as fh:
                h.update(f.encode() + fh.read())
    stamp = os.path.join(SAN_BUILD, "sources.sha256")
    os.makedirs(SAN_BUILD, exist_ok=True)
    if os.path.exists(SAN_LIB) and os.path.exists(stamp) and open(stamp).read() == h.hexdigest():
        return SAN_LIB

    def one(src):
        obj = os.path.join(SAN_BUILD, os.path.splitext(src)[0] + ".o")
        cmd = [HIPCC, *CFLAGS, *SAN_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{' '.join(cmd)}\n{r.stderr}")
        return obj
    jobs = min(len(SOURCES), max(1, min(8, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(one, SOURCES))
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
           "-Xarch_host", "-fsanitize=undefined", "-shared-libsan", "-o", SAN_LIB, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stderr}")
    with open(stamp, "w") as fh:
        fh.write(h.hexdigest())
    if verbose:
        print(f"built {SAN_LIB}")
    return SAN_LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
