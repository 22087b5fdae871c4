"""Builds libforge.so (the gfx950 HIP kernels + C ABI) in-tree with hipcc.

Usage: python optimizer_gemm_amd/build.py   (or __graft_entry__.build()); run by path,
since importing the package loads the library this script builds.
The library lands in optimizer_gemm_amd/_lib/libforge.so; object files in
optimizer_gemm_amd/_build/. Every call recompiles.

python optimizer_gemm_amd/build.py --sanitize builds the host-checking variant,
optimizer_gemm_amd/_build/san/libforge_san.so: AddressSanitizer and
UndefinedBehaviorSanitizer on the host code only (each flag behind -Xarch_host; the
device code is the release build's). A process loads it with the sanitizer runtime
first, LD_PRELOAD=$(sanitizer runtime) FORGE_LIB=.../libforge_san.so, and
ASAN_OPTIONS=detect_leaks=0 (the interpreter keeps its allocations to the end).
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
BUILD = os.path.join(PKG, "_build")
LIBDIR = os.path.join(PKG, "_lib")
LIB = os.path.join(LIBDIR, "libforge.so")
ARCH = os.environ.get("FORGE_OFFLOAD_ARCH", "gfx950")

# every HIP source of csrc/ (the fused-step instantiations are split over several
# files so they compile in parallel)
SOURCES = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))

CFLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # packed fp32 VALU forms are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
    "-I", os.path.join(ROOT, "include"),
]


def _hipcc() -> str:
    h = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(h):
        raise RuntimeError("hipcc not found; the forge library needs ROCm's hipcc")
    return h


# host-checking variant: sanitizers on the host pass only
SAN_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
            "-Xarch_host", "-g"]
SAN_LINK = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-shared-libasan"]
SAN_DIR = os.path.join(BUILD, "san")
SAN_LIB = os.path.join(SAN_DIR, "libforge_san.so")
# the compiler's per-kernel register / LDS / scratch report, printed on stderr
REMARKS = ["-Rpass-analysis=kernel-resource-usage"]


def _compile(src: str, out_dir: str = BUILD, extra=()) -> tuple:
    obj = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc(), *CFLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj, r.stderr


def _link(objs, out: str, extra=()) -> str:
    tmp = out + ".tmp"
    # -z defs: a kernel whose host-side launch stub was not emitted would otherwise
    # link into a library that fails only when it is loaded
    cmd = [_hipcc(), "-shared", f"--offload-arch={ARCH}", *extra, "-Wl,-z,defs", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    return out


def _compile_all(out_dir: str, extra=()) -> list:
    os.makedirs(out_dir, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        return list(ex.map(lambda s: _compile(s, out_dir, extra), SOURCES))


def build(verbose: bool = False) -> str:
    os.makedirs(LIBDIR, exist_ok=True)
    objs = [o for o, _ in _compile_all(BUILD)]
    _link(objs, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


def build_sanitized(remarks: bool = False, verbose: bool = False) -> tuple:
    """The host-checking variant (module docstring): (library path, {source: compiler
    stderr}); with remarks=True that stderr holds every kernel's resource report."""
    res = _compile_all(SAN_DIR, SAN_HOST + (REMARKS if remarks else []))
    _link([o for o, _ in res], SAN_LIB, SAN_LINK)
    if verbose:
        print(f"built {SAN_LIB}")
    return SAN_LIB, {src: err for src, (_, err) in zip(SOURCES, res)}


def sanitizer_runtime() -> str:
    """Path of the AddressSanitizer runtime the host-checking variant links against."""
    clang = os.path.join(os.path.dirname(os.path.realpath(_hipcc())), "..", "llvm", "bin", "clang++")
    for c in (clang, "/opt/rocm/llvm/bin/clang++", shutil.which("clang++") or ""):
        if c and os.path.exists(c):
            p = subprocess.run([c, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                               text=True).stdout.strip()
            if os.path.isabs(p) and os.path.exists(p):
                return p
    raise RuntimeError("AddressSanitizer runtime (libclang_rt.asan-x86_64.so) not found")


if __name__ == "__main__":
    if "--sanitize" in sys.argv[1:]:
        build_sanitized(verbose=True)
    else:
        build(verbose=True)
    sys.exit(0)
