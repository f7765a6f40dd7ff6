"""Build libqkrope.so: the HIP kernel family and the C ABI, for gfx950; and _qkrope_native, the
C++ marshalling of the two page signatures onto that C ABI (host code, built with g++ against
torch's headers).

The library links against the HIP runtime that PyTorch loads (torch/lib/libamdhip64.so), so a
process that uses torch for memory and streams has exactly one HIP runtime, and the hipStream_t
handles torch gives out are valid inside the library.
"""
from __future__ import annotations

import os
import subprocess
import sys
import sysconfig
import time
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(PKG, "libqkrope.so")
NATIVE_SRC = os.path.join(PKG, "qkrope_native.cpp")
NATIVE_PATH = os.path.join(PKG, "_qkrope_native" + sysconfig.get_config_var("EXT_SUFFIX"))

SOURCES = ["qkrope_kernels_3d_d64.hip", "qkrope_kernels_3d_d128.hip", "qkrope_kernels_3d_d256.hip",
           "qkrope_kernels_table_interleaved_bf16.hip", "qkrope_kernels_table_halfsplit_bf16.hip",
           "qkrope_kernels_table_interleaved_f16.hip", "qkrope_kernels_table_halfsplit_f16.hip",
           "qkrope_kernels_table_halfsplit_any_bf16.hip", "qkrope_kernels_table_halfsplit_any_f16.hip",
           "qkrope_kernels_sumsq.hip", "qkrope_kernels_cam.hip", "qkrope_api.cpp",
           "qkrope_api_cam.cpp"]

HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # no packed-fp32 VALU forms in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]


def torch_lib_dir() -> str:
    import torch
    return os.path.join(os.path.dirname(torch.__file__), "lib")


def native_compile_cmd(obj: str) -> list:
    """g++ line for the page-signature marshaller: torch's headers and ABI settings (the
    pybind11 ABI tags torch was built with, so its tensor type casters are shared)."""
    import torch
    tdir = os.path.dirname(torch.__file__)
    flags = [f"-D_GLIBCXX_USE_CXX11_ABI={int(torch._C._GLIBCXX_USE_CXX11_ABI)}"]
    for name in ("COMPILER_TYPE", "STDLIB", "BUILD_ABI"):
        val = getattr(torch._C, f"_PYBIND11_{name}", None)
        if val is not None:
            flags.append(f'-DPYBIND11_{name}="{val}"')
    return ["g++", "-O2", "-std=c++17", "-fPIC", "-w", "-D__HIP_PLATFORM_AMD__", "-DUSE_ROCM",
            *flags, "-I", os.path.join(tdir, "include"),
            "-I", os.path.join(tdir, "include", "torch", "csrc", "api", "include"),
            "-I", sysconfig.get_paths()["include"], "-I", "/opt/rocm/include", "-I", INCLUDE,
            "-c", NATIVE_SRC, "-o", obj]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "is not a recognized feature for this target" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if out.strip() and verbose:
        print(out, flush=True)


def build(verbose: bool = True) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    os.makedirs(BUILD_DIR, exist_ok=True)
    t0 = time.time()
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmds.append([hipcc, *HIP_FLAGS, "-I", INCLUDE, "-I", CSRC, *lang, "-c",
                     os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    native_obj = os.path.join(BUILD_DIR, "qkrope_native.o")
    cmds.append(native_compile_cmd(native_obj))
    with ThreadPoolExecutor(max_workers=len(cmds)) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    tlib = torch_lib_dir()
    tmp = LIB_PATH + ".tmp"
    _run(["g++", "-shared", "-o", tmp, *objs, f"-L{tlib}", "-l:libamdhip64.so",
          f"-Wl,-rpath,{tlib}", "-Wl,--no-undefined"], verbose)
    os.replace(tmp, LIB_PATH)
    # the marshaller links the library it calls (found next to it at run time) and torch's
    tmp = NATIVE_PATH + ".tmp"
    _run(["g++", "-shared", "-o", tmp, native_obj, f"-L{PKG}", "-l:libqkrope.so",
          "-Wl,-rpath,$ORIGIN", f"-L{tlib}", "-lc10", "-ltorch", "-ltorch_cpu", "-ltorch_python",
          "-lc10_hip", f"-Wl,-rpath,{tlib}"], verbose)
    os.replace(tmp, NATIVE_PATH)
    if verbose:
        print(f"built {LIB_PATH} and {NATIVE_PATH} in {time.time() - t0:.1f}s", flush=True)
    return LIB_PATH


if __name__ == "__main__":
    build(verbose="-q" not in sys.argv)
