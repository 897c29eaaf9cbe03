"""Build libvjsd.so in-tree with hipcc for gfx950.

Every HIP source is compiled (in parallel) to an object under ``_build/`` and
linked into ``vocab_sharded_softmax_amd/libvjsd.so``.  Packed fp32 vector
instructions are disabled for the device code; the host pass warns that it does
not know that target feature, which is harmless.
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
OBJ = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libvjsd.so")
SOURCES = ["api.hip", "stats.hip", "jsd.hip", "fused.hip", "siblings.hip", "probe.hip", "reduce.hip", "gemm.hip", "linear.hip"]
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    # no implicit fused multiply-adds: the kernels rely on products being rounded
    # exactly where the source rounds them, and write every FMA explicitly
    "-ffp-contract=off",
    "-Wall", "-Wno-unused-function", "-Wno-unused-result",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libvjsd")


def _compile(src: str) -> str:
    out = os.path.join(OBJ, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *FLAGS, "-c", os.path.join(CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines()
            if "packed-fp32-ops" not in ln or "error" in ln]
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n" + "\n".join(msgs))
    if msgs:
        sys.stderr.write("\n".join(msgs) + "\n")
    return out


def build(jobs: int = 4) -> str:
    """Compile every HIP source and link libvjsd.so; returns its path."""
    os.makedirs(OBJ, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link of libvjsd.so failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    return LIB


# Host-side AddressSanitizer and UndefinedBehaviorSanitizer for the C ABI's argument
# checks (csrc/api.hip): each sanitizer flag applies to the host pass only, the device
# code is compiled as usual.  Loaded with the clang ASan runtime preloaded (it carries
# the UBSan handlers too).
SAN_FLAGS = ["-O1", "-g", "-Xarch_host", "-fsanitize=address", "-Xarch_host",
             "-fsanitize=undefined", "-Xarch_host", "-fno-sanitize-recover=undefined",
             "-Xarch_host", "-fno-omit-frame-pointer"]
SAN_DIR = os.path.join(OBJ, "san")


def build_host_sanitized() -> str:
    """libvjsd with api.hip's host code under ASan + UBSan (the other objects as built
    by build()); returns the library's path, _build/san/libvjsd_san.so."""
    if not all(os.path.exists(os.path.join(OBJ, os.path.splitext(x)[0] + ".o")) for x in SOURCES):
        build()
    os.makedirs(SAN_DIR, exist_ok=True)
    flags = [f for f in FLAGS if f != "-O3"] + SAN_FLAGS
    api_o = os.path.join(SAN_DIR, "api.o")
    r = subprocess.run([hipcc(), *flags, "-c", os.path.join(CSRC, "api.hip"), "-o", api_o],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("sanitized build of api.hip failed:\n" + r.stdout + r.stderr)
    objs = [os.path.join(OBJ, os.path.splitext(x)[0] + ".o") for x in SOURCES if x != "api.hip"]
    lib = os.path.join(SAN_DIR, "libvjsd_san.so")
    r = subprocess.run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", lib, *objs,
                        api_o], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link of libvjsd_san.so failed:\n" + r.stdout + r.stderr)
    return lib


def asan_runtime() -> str:
    """The clang ASan runtime of the HIP toolchain (to preload for build_host_sanitized's
    library)."""
    import glob

    root = os.path.dirname(os.path.dirname(os.path.realpath(hipcc())))
    for pat in ("llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so",
                "llvm/lib/clang/*/lib/x86_64-unknown-linux-gnu/libclang_rt.asan.so"):
        hits = sorted(glob.glob(os.path.join(root, pat)))
        if hits:
            return hits[-1]
    raise RuntimeError("clang ASan runtime not found under " + root)


if __name__ == "__main__":
    print(build())
