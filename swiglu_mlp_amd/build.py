"""Build libdfk.so (HIP kernels + C-ABI runtime) in-tree for gfx950.

    python -m swiglu_mlp_amd.build

hipcc cross-compiles for gfx950 without a GPU.  The library lands next to
this file (swiglu_mlp_amd/libdfk.so); the tuning table it reads by default is
swiglu_mlp_amd/tuning/gfx950.json.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIBRARY = os.path.join(PKG, "libdfk.so")
ARCH = "gfx950"

# -packed-fp32-ops: keep the compiler from emitting v_pk_{add,mul,fma}_f32.
HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}", f"-I{CSRC}",
]
SOURCES = ["dfk_kernels.hip", "dfk_stream.hip", "dfk_runtime.cpp"]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: the ROCm toolchain is required to build libdfk.so")
    return path


def _compile(src: str, defines=(), build_dir: str = BUILD_DIR) -> str:
    os.makedirs(build_dir, exist_ok=True)
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *HIP_FLAGS, *[f"-D{d}" for d in defines], "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        # host-only runtime: plain C++ against the HIP runtime headers
        cmd = [hipcc(), "-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra", f"-I{INCLUDE}", f"-I{CSRC}",
               "-D__HIP_PLATFORM_AMD__", "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def build(verbose: bool = False, output: str = LIBRARY, defines=(), build_dir: str = BUILD_DIR) -> str:
    """Compile every source and link the library; returns its path.  `defines`
    (NAME=VALUE strings) override the kernels' compile-time tile parameters."""
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as pool:
        objs = list(pool.map(lambda s: _compile(s, defines, build_dir), SOURCES))
    tmp = output + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp, "-ldl"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stderr}")
    os.replace(tmp, output)
    if verbose:
        print(f"built {output}")
    return output


# Host-side sanitizer build: the C-ABI runtime (host C++ only) compiled with
# g++ under AddressSanitizer and UndefinedBehaviorSanitizer, linked with the
# regular HIP objects (GPU code is never built with a sanitizer).  Load it
# with DFK_LIBRARY and libasan preloaded; for the CPU-side tests.
SANITIZE = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined"]


def build_host_sanitized(output: str, build_dir: str = BUILD_DIR) -> str:
    """Link libdfk with an ASan/UBSan-instrumented runtime; returns the path.
    The kernel objects come from `build_dir` (built first when missing)."""
    os.makedirs(build_dir, exist_ok=True)
    kernel_objs = []
    for src in SOURCES:
        if src.endswith(".cpp"):
            continue
        obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
        if not os.path.exists(obj):
            obj = _compile(src, (), build_dir)
        kernel_objs.append(obj)
    rt = os.path.join(os.path.dirname(os.path.abspath(output)), "dfk_runtime_san.o")
    cc = ["g++", "-O1", "-g", "-fno-omit-frame-pointer", *SANITIZE, "-std=c++17", "-fPIC", "-Wall", "-Wextra",
          "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", f"-I{INCLUDE}", f"-I{CSRC}",
          "-c", os.path.join(CSRC, "dfk_runtime.cpp"), "-o", rt]
    res = subprocess.run(cc, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cc)}\n{res.stderr}")
    ld = ["g++", "-shared", *SANITIZE, rt, *kernel_objs, "-L/opt/rocm/lib", "-Wl,-rpath,/opt/rocm/lib",
          "-lamdhip64", "-ldl", "-o", output]
    res = subprocess.run(ld, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(ld)}\n{res.stderr}")
    return output


if __name__ == "__main__":
    build(verbose=True)
