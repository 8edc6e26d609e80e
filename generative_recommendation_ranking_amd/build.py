"""Builds libmtgr.so for gfx950 with hipcc (cross-compiles; no GPU needed).

    python -m generative_recommendation_ranking_amd.build [--sanitize]

Each HIP source compiles to its own object in parallel, then one shared library is linked next to
this file, where the binding loads it.  Packed fp32 instructions are switched off for device code.

--sanitize builds a second copy, _build_san/libmtgr_san.so, whose host code (argument checks,
workspace planning, launch sequencing) carries the address and undefined-behaviour sanitizers;
device code is compiled as usual.  Load it with MTGR_LIB pointing at it and the compiler's ASan
runtime preloaded (sanitizer_runtime() gives its path); tests/test_host_plan.py does this for the
host-side ABI checks.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(PKG, "_build")
LIB_PATH = os.path.join(PKG, "libmtgr.so")
SAN_DIR = os.path.join(PKG, "_build_san")
SAN_LIB_PATH = os.path.join(SAN_DIR, "libmtgr_san.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libmtgr.so)")


COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


# host-side sanitizers only (each flag behind -Xarch_host, so device code is built as usual)
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address,undefined", "-Xarch_host", "-fno-omit-frame-pointer",
             "-Xarch_host", "-fno-sanitize-recover=undefined", "-shared-libasan"]


def sanitizer_runtime() -> str:
    """path of the compiler's shared ASan runtime, to preload into a process that loads the
    sanitized library"""
    out = subprocess.run([hipcc(), "--print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                         text=True).stdout.strip()
    if not out or not os.path.exists(out):
        import glob
        found = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
        out = found[0] if found else ""
    if not out:
        raise RuntimeError("the compiler's ASan runtime was not found")
    return out


def _compile(src: str, out_dir: str = BUILD_DIR, extra=()) -> str:
    obj = os.path.join(out_dir, os.path.basename(src)[:-4] + ".o")
    cmd = [hipcc(), *COMMON_FLAGS, *extra, "-I", INCLUDE, "-I", CSRC, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build_library(verbose: bool = False, sanitize: bool = False) -> str:
    out_dir, lib_path = (SAN_DIR, SAN_LIB_PATH) if sanitize else (BUILD_DIR, LIB_PATH)
    extra = SAN_FLAGS if sanitize else []
    os.makedirs(out_dir, exist_ok=True)
    srcs = sources()
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s_: _compile(s_, out_dir, extra), srcs))
    tmp = lib_path + ".tmp"
    # -z defs: a kernel whose host stub was not emitted fails here, not at load time (the sanitized
    # copy resolves its runtime from the preloaded ASan library instead)
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *(extra or ["-Wl,-z,defs"]), *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, lib_path)
    if verbose:
        print(f"built {lib_path}")
    return lib_path


if __name__ == "__main__":
    build_library(verbose=True, sanitize="--sanitize" in sys.argv[1:])
    sys.exit(0)
