"""Build the PISA HIP library in-tree: block_sparse_long_pisa_amd/lib/libpisa.so (gfx950).

Usage: python -m block_sparse_long_pisa_amd.build [--jobs N]
"""

from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(ROOT, "_build", "obj")
LIB = os.path.join(PKG, "lib", "libpisa.so")
SOURCES = ["pisa_api.hip", "pisa_pool.hip", "pisa_select.hip", "pisa_attn.hip", "pisa_attn_bwd.hip", "pisa_decode.hip",
           "pisa_fused.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the PISA library needs the ROCm toolchain")


def compile_flags():
    return [
        f"--offload-arch={ARCH}",
        "-O3",
        "-std=c++17",
        "-fPIC",
        "-Wall",
        "-Wno-unused-function",
        "-Wno-unused-variable",
        # no packed fp32 instructions in device code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        f"-I{INCLUDE}",
        f"-I{CSRC}",
    ]


def _compile(src: str) -> str:
    obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *compile_flags(), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(jobs: int = 5, verbose: bool = False) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    os.makedirs(os.path.dirname(LIB), exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


# Host-sanitised build of the C-ABI validation (pisa_api.hip, with AddressSanitizer
# and UndefinedBehaviorSanitizer on its host code only), linked with the normal
# objects of the other sources. Loaded through PISA_LIBRARY into a process whose
# sanitizer runtime is preloaded; it runs the host-side argument checks under the
# sanitizers (no kernel is launched by those checks).
SAN_LIB = os.path.join(ROOT, "_build", "san", "libpisa_san.so")
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def sanitizer_runtime() -> str:
    """Path of the AddressSanitizer runtime that the host-sanitised library needs preloaded."""
    r = subprocess.run([os.path.join(os.path.dirname(hipcc()), "..", "llvm", "bin", "clang++"),
                        "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.exists(path):
        raise RuntimeError("the AddressSanitizer runtime of the ROCm toolchain was not found")
    return path


def build_sanitized(verbose: bool = False) -> str:
    san_dir = os.path.dirname(SAN_LIB)
    os.makedirs(san_dir, exist_ok=True)
    objs = []
    for src in SOURCES:
        if src == "pisa_api.hip":
            obj = os.path.join(san_dir, "pisa_api.o")
            cmd = [hipcc(), *compile_flags(), *SAN_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
            r = subprocess.run(cmd, capture_output=True, text=True)
            if r.returncode != 0:
                raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
        else:
            obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
            if not os.path.exists(obj):
                obj = _compile(src)
        objs.append(obj)
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *SAN_FLAGS, "-shared-libsan", "-o", SAN_LIB, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    if verbose:
        print(f"built {SAN_LIB}")
    return SAN_LIB


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=5)
    ap.add_argument("--sanitized", action="store_true", help="build the host-sanitised library instead")
    a = ap.parse_args(argv)
    if a.sanitized:
        build_sanitized(verbose=True)
    else:
        build(a.jobs, verbose=True)


if __name__ == "__main__":
    sys.exit(main())
