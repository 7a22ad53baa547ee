"""Build libh2o.so (HIP, gfx950) in-tree: h2o_sparse_attention_amd/lib/libh2o.so.

Usage: python h2o_sparse_attention_amd/build.py [--verbose]
(run as a file: importing the package loads the library this script builds)
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OBJ_DIR = os.path.join(HERE, "_build")
LIB_DIR = os.path.join(HERE, "lib")
LIB_PATH = os.path.join(LIB_DIR, "libh2o.so")

SOURCES = ["api.hip", "attn_bf16.hip", "attn_f32.hip", "attn_bwd.hip", "evict.hip", "decode.hip",
           "noalloc.hip"]
ARCH = "gfx950"
CXXFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    "-Wall", "-Wno-unused-function",
    # no packed fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # the host pass does not know the packed-fp32 target feature; that warning is expected
    out = "\n".join(l for l in p.stdout.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if p.returncode != 0:
        raise RuntimeError(f"command failed ({p.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out)


def build(verbose: bool = False) -> str:
    """Compile every HIP source for gfx950 and link libh2o.so; return its path."""
    hipcc = _hipcc()
    os.makedirs(OBJ_DIR, exist_ok=True)
    os.makedirs(LIB_DIR, exist_ok=True)
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(OBJ_DIR, src.replace(".hip", ".o"))
        objs.append(obj)
        cmds.append([hipcc, *CXXFLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(cmds))) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    tmp = LIB_PATH + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


# Host-side AddressSanitizer + UndefinedBehaviorSanitizer, on the host pass only (the
# device code is built as usual); the runtime is linked as a shared library, which the
# process that loads this build must preload (clang -print-file-name gives its path).
HOST_SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"]


def asan_runtime() -> str:
    """Path of the shared ASan runtime of ROCm's clang (it carries the UBSan handlers too)."""
    clang = os.path.join(os.path.dirname(os.path.realpath(_hipcc())), "..", "lib", "llvm",
                         "bin", "clang")
    if not os.path.exists(clang):
        clang = "/opt/rocm/llvm/bin/clang"
    out = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"],
                         stdout=subprocess.PIPE, text=True, check=True).stdout.strip()
    if not os.path.isabs(out) or not os.path.exists(out):
        raise RuntimeError(f"ASan runtime not found (clang printed {out!r})")
    return out


def build_host_sanitized(out_dir: str, verbose: bool = False) -> str:
    """Build the same sources into out_dir/libh2o_san.so with the host code under ASan and
    UBSan (-O1 -g, frame pointers kept); return its path. Loading it needs the ASan
    runtime preloaded (LD_PRELOAD=asan_runtime())."""
    hipcc = _hipcc()
    os.makedirs(out_dir, exist_ok=True)
    flags = [f for f in CXXFLAGS if f != "-O3"] + ["-O1", "-g", "-fno-omit-frame-pointer"]
    objs, cmds = [], []
    for src in SOURCES:
        obj = os.path.join(out_dir, src.replace(".hip", ".san.o"))
        objs.append(obj)
        cmds.append([hipcc, *flags, *HOST_SAN_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(cmds))) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    lib = os.path.join(out_dir, "libh2o_san.so")
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-shared-libsan", *HOST_SAN_FLAGS,
          "-o", lib, *objs], verbose)
    return lib


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
