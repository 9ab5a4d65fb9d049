"""Build the HIP library in-tree: image_dit_amd/libsparse_attn.so (gfx950).

Usage: python -m image_dit_amd.build   (always recompiles every source)
"""

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libsparse_attn.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["api.cpp", "planner.cpp", "permute.hip", "predict.hip", "flash.hip", "noalloc.hip", "quant.hip"]

COMMON = ["-O3", "-fPIC", "-std=c++17", f"--offload-arch={ARCH}",
          "-I", os.path.join(ROOT, "include"), "-I", CSRC,
          # no packed fp32 VALU ops in device code
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wno-unused-command-line-argument"]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *COMMON, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    # a kernel template whose host-side instantiation failed leaves its launch
    # stub undefined without any diagnostic: refuse such a library
    nm = subprocess.run(["nm", "-D", "--undefined-only", tmp], capture_output=True, text=True)
    missing = [l.split()[-1] for l in nm.stdout.splitlines() if "device_stub" in l]
    if missing:
        os.remove(tmp)
        raise RuntimeError("kernel launch stubs missing from the library: " + ", ".join(missing))
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    _build_example(verbose)
    return LIB


DEMO = os.path.join(BUILD, "path_demo")


def _build_example(verbose: bool) -> None:
    """The plain-C caller of the whole path (examples/path_demo.c), linked against the
    library through $ORIGIN so the pair can move together."""
    gcc = shutil.which("gcc")
    if gcc is None:
        if verbose:
            print("gcc not found: examples/path_demo.c not built")
        return
    rocm = os.path.dirname(os.path.dirname(os.path.realpath(HIPCC)))
    cmd = [gcc, "-std=c99", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-isystem", os.path.join(rocm, "include"),
           os.path.join(PKG, "examples", "path_demo.c"), "-L", PKG, "-lsparse_attn",
           "-L", os.path.join(rocm, "lib"), "-lamdhip64", "-Wl,-rpath,$ORIGIN/..",
           "-Wl,-rpath," + os.path.join(rocm, "lib"), "-o", DEMO]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"gcc failed on examples/path_demo.c:\n{r.stdout}\n{r.stderr}")
    if verbose:
        print(f"built {DEMO}")


if __name__ == "__main__":
    build()
    sys.exit(0)
