"""Build libmok.so (the gfx950 HIP library) in-tree with hipcc.

Every HIP source is compiled for gfx950 only, with packed-fp32 instructions
disabled (``-Xclang -target-feature -Xclang -packed-fp32-ops``), and linked
into ``combine_router_top_expert_amd/libmok.so`` next to this file.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmok.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


# Host-side AddressSanitizer + UndefinedBehaviorSanitizer build (the device
# code is compiled as usual; every sanitizer flag applies to the host pass
# only).  It runs the host logic -- argument checks, workspace layout, table
# marshalling -- on the CPU; the process must preload the sanitizer runtime
# that SANITIZER_RUNTIME names.
SAN_FLAGS = ["-g", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def sanitizer_runtime() -> str:
    """The clang AddressSanitizer runtime (it carries the UB handlers too)."""
    hits = sorted(glob.glob(os.path.join(os.path.dirname(os.path.dirname(HIPCC)), "llvm", "lib",
                                         "clang", "*", "lib", "linux",
                                         "libclang_rt.asan-x86_64.so")))
    if not hits:
        raise RuntimeError("no clang AddressSanitizer runtime next to hipcc")
    return hits[-1]


def _compile(src: str, build_dir: str = BUILD, extra=()) -> str:
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False, out: str = LIB, sanitize: bool = False) -> str:
    build_dir = os.path.join(os.path.dirname(out), "_build_san") if sanitize else BUILD
    extra = SAN_FLAGS if sanitize else []
    os.makedirs(build_dir, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, build_dir, extra), srcs))
    tmp = out + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC"]
    if sanitize:
        cmd += ["-shared-libsan", "-Xarch_host", "-fsanitize=address", "-Xarch_host",
                "-fsanitize=undefined"]
    cmd += ["-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    if verbose:
        print("built", out)
    return out


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
