"""Build librq.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python -m gemm_rwkv_amd.build          # compiles every source, always

Each source is compiled to an object under ``_build/`` in parallel, then the
objects are linked into ``gemm_rwkv_amd/librq.so``.  Packed fp32 VALU
instructions are disabled for all device code.
"""

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "librq.so")

SOURCES = ["api.hip", "quant.hip", "gemv.hip", "gemm_mfma.hip", "gemm_w4.hip", "measure.hip", "validate.cpp",
           "proxy.cpp"]
ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + INCLUDE, "-I" + CSRC,
]


# per-source options: the dense GEMM keeps its accumulators in VGPRs (with
# them in AGPRs the allocator shuttles them between the two files every
# k step of the double-buffered loop)
EXTRA = {"gemm_mfma.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src):
    obj = os.path.join(BUILD, src + ".o")
    cmd = [HIPCC] + FLAGS + EXTRA.get(src, []) + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("compile failed: %s\n%s\n%s" % (" ".join(cmd), r.stdout, r.stderr))
    return obj


def build(verbose=True):
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), 8)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed: %s\n%s" % (r.stdout, r.stderr))
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


SANITIZED = os.path.join(BUILD, "sanitized", "librq.so")
# host-side sanitizers only (device code is built as usual)
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=all"]
HOST_SOURCES = ["api.hip", "validate.cpp", "proxy.cpp"]


def build_sanitized(verbose=True):
    """librq.so with the host-side C ABI layer (argument validation, planning
    inputs) built under AddressSanitizer and UndefinedBehaviorSanitizer, linked
    with the kernel objects of the regular build, at _build/sanitized/.  Load
    it with the sanitizer runtime preloaded (see tests/test_abi_sanitized.py)."""
    out = os.path.dirname(SANITIZED)
    os.makedirs(out, exist_ok=True)
    kernel_objs = [os.path.join(BUILD, src + ".o") for src in SOURCES if src not in HOST_SOURCES]
    if not all(os.path.exists(o) for o in kernel_objs):
        build(verbose)
    objs = []
    for src in HOST_SOURCES:
        obj = os.path.join(out, src + ".o")
        cmd = [HIPCC] + FLAGS + SAN_FLAGS + ["-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("compile failed: %s\n%s\n%s" % (" ".join(cmd), r.stdout, r.stderr))
        objs.append(obj)
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-fsanitize=address,undefined", "-shared-libsan",
           "-o", SANITIZED] + objs + kernel_objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed: %s\n%s" % (r.stdout, r.stderr))
    if verbose:
        print("built", SANITIZED)
    return SANITIZED


def sanitizer_runtime():
    """Path of the clang AddressSanitizer runtime the sanitized build links."""
    r = subprocess.run([HIPCC, "--print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        import glob
        cands = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
        path = cands[0] if cands else ""
    return path


if __name__ == "__main__":
    if len(sys.argv) > 1 and sys.argv[1] == "sanitized":
        build_sanitized()
    else:
        build()
    sys.exit(0)
