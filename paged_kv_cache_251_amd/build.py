"""Build libpagedattn.so in-tree with hipcc for gfx950.

    python -m paged_kv_cache_251_amd.build              # libpagedattn.so
    python -m paged_kv_cache_251_amd.build --sanitize   # libpagedattn_san.so
    python -m paged_kv_cache_251_amd.build --define NAME=VALUE ... --out PATH
        # a comparison build with the sources' tuning switches set (e.g.
        # PA_DECODE_MFMA_WIDE_GROUPS=0: the vector decode pass for every group size), written to
        # PATH and loaded with PA_LIBRARY=PATH; its objects go to a folder of their own

The sanitized library has its host code (the C ABI, the block manager, the scheduler) built with
AddressSanitizer and UndefinedBehaviorSanitizer (host side only; the kernels are built as usual).
It is loaded in place of the plain one with PA_LIBRARY=<path> and the sanitizer runtime preloaded
(sanitizer_env() gives the environment); tests/test_sanitize_cpu.py runs the host-side tests that
way.
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
LIB = os.path.join(PKG, "libpagedattn.so")
OBJ_SAN = os.path.join(PKG, "_build_san")
LIB_SAN = os.path.join(PKG, "libpagedattn_san.so")
HOST_SOURCES = ("api.cpp", "block_manager.cpp", "scheduler.cpp")
# host-side sanitizers; every -fsanitize flag applies to the host compilation only
SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
            "-Xarch_host", "-g"]

SOURCES = ["api.cpp", "block_manager.cpp", "scheduler.cpp", "cache_write.hip", "decode.hip", "reduce.hip", "varlen.hip",
           "multiquery.hip", "packed.hip"]
ARCH = os.environ.get("PA_OFFLOAD_ARCH", "gfx950")

FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-result",
    "-munsafe-fp-atomics",
    # never emit packed fp32 arithmetic (v_pk_{add,mul,fma}_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}",
    f"-I{CSRC}",
]


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def _compile(src: str, verbose: bool, sanitize: bool = False, defines=(), obj=None) -> str:
    out = os.path.join(obj or (OBJ_SAN if sanitize else OBJ), os.path.splitext(src)[0] + ".o")
    extra = SANITIZE if sanitize and src in HOST_SOURCES else []
    cmd = [_hipcc(), *FLAGS, *extra, *(f"-D{d}" for d in defines), "-c", os.path.join(CSRC, src), "-o", out]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{msg}")
    if verbose and msg.strip():
        print(msg, flush=True)
    return out


def build(verbose: bool = False, sanitize: bool = False, defines=(), out=None) -> str:
    """Compile and link the library.  `defines` (NAME=VALUE strings) and `out` make a comparison
    build: it never replaces the plain library and keeps its objects apart."""
    if defines and not out:
        raise ValueError("a build with defines needs an output path of its own")
    obj = None
    if out:
        import hashlib

        tag = hashlib.sha1(" ".join(sorted(defines)).encode()).hexdigest()[:10]
        obj = os.path.join(PKG, f"_build_{tag}")
    os.makedirs(obj or (OBJ_SAN if sanitize else OBJ), exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, sanitize, defines, obj), SOURCES))
    lib = os.path.abspath(out) if out else (LIB_SAN if sanitize else LIB)
    tmp = lib + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, lib)
    return lib


def sanitizer_runtime() -> str:
    """The compiler's shared AddressSanitizer runtime (it carries the UndefinedBehaviorSanitizer
    handlers too)."""
    r = subprocess.run([_hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path):
        return path
    import glob

    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/*/libclang_rt.asan-x86_64.so"))
    if not found:
        raise RuntimeError("libclang_rt.asan-x86_64.so not found")
    return found[-1]


def sanitizer_env(base=None) -> dict:
    """Environment for a host-only process that loads the sanitized library through the binding."""
    env = dict(os.environ if base is None else base)
    env["PA_LIBRARY"] = LIB_SAN
    env["LD_PRELOAD"] = sanitizer_runtime()
    # the interpreter itself is not instrumented: its own allocations are not leak-checked
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    return env


if __name__ == "__main__":
    import argparse

    ap = argparse.ArgumentParser()
    ap.add_argument("-v", action="store_true", dest="verbose")
    ap.add_argument("--sanitize", action="store_true")
    ap.add_argument("--define", action="append", default=[], metavar="NAME=VALUE")
    ap.add_argument("--out", default=None, metavar="PATH")
    a = ap.parse_args()
    print(build(verbose=a.verbose, sanitize=a.sanitize, defines=a.define, out=a.out))
