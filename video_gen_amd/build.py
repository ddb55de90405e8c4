"""Build libbasa.so (HIP, gfx950) in-tree with hipcc.

Every source under ``csrc/`` is compiled as HIP for gfx950 only and linked into
``video_gen_amd/libbasa.so``.  Packed-FP32 instructions are disabled for all
device code.  Run ``python -m video_gen_amd.build`` or ``__graft_entry__.build()``.

``build(sanitize=True)`` (``python -m video_gen_amd.build --sanitize``) makes a
second copy under ``_build/libbasa_san/`` whose host code (plan, argument
checks, launch set-up) is instrumented with AddressSanitizer and
UndefinedBehaviorSanitizer; device code is compiled as usual.  The
instrumented library resolves the sanitizer runtime at load time, so the
process that loads it preloads clang's ``libclang_rt.asan`` (see
``sanitizer_runtime()``).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libbasa.so")
BUILD_DIR = os.path.join(os.path.dirname(PKG), "_build", "libbasa")
SAN_DIR = os.path.join(os.path.dirname(PKG), "_build", "libbasa_san")
SAN_OUT = os.path.join(SAN_DIR, "libbasa.so")
ARCH = "gfx950"
SOURCES = ["plan.cpp", "api.cpp", "k_index.hip", "k_pool.hip", "k_route.hip", "k_attn.hip",
           "k_bwd.hip", "k_merge.hip", "k_probe.hip"]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise FileNotFoundError("hipcc not found (ROCm is required to build libbasa)")


def compile_flags() -> list:
    return [
        "-x", "hip", f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        "-Wall", "-Wno-unused-function",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        f"-I{os.path.join(os.path.dirname(PKG), 'include')}",
    ]


# Host-only instrumentation: every sanitizer flag is scoped to the host pass.
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined",
             "-Xarch_host", "-fno-omit-frame-pointer"]


def sanitizer_runtime() -> str:
    """Path of clang's shared ASan runtime (it also carries the UBSan handlers)."""
    import glob

    root = os.path.dirname(os.path.dirname(os.path.realpath(hipcc())))
    hits = sorted(glob.glob(os.path.join(root, "llvm", "lib", "clang", "*", "lib", "linux",
                                         "libclang_rt.asan-x86_64.so")))
    if not hits:
        raise FileNotFoundError("libclang_rt.asan-x86_64.so not found under the ROCm LLVM")
    return hits[-1]


# Extra flags per source.  The attention kernel never sees NaN inputs it must
# propagate (scores are finite or -inf), so fmax lowers to plain v_max/v_max3.
EXTRA = {"k_attn.hip": ["-fno-honor-nans"]}


def _compile(src: str, verbose: bool, sanitize: bool = False) -> str:
    obj = os.path.join(SAN_DIR if sanitize else BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *compile_flags(), *EXTRA.get(src, []), *(SAN_FLAGS if sanitize else []),
           "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    if verbose and r.stderr.strip():
        print(r.stderr, file=sys.stderr)
    return obj


def build(verbose: bool = False, sanitize: bool = False) -> str:
    """Compile every HIP source and link libbasa.so; returns its path.

    sanitize: build the host-instrumented copy under ``_build/libbasa_san``
    instead of the in-tree library.
    """
    out = SAN_OUT if sanitize else OUT
    os.makedirs(SAN_DIR if sanitize else BUILD_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, sanitize), SOURCES))
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp,
           "-Wl,-rpath,/opt/rocm/lib"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link of libbasa.so failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True, sanitize="--sanitize" in sys.argv[1:]))
