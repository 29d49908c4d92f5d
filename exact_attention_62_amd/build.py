"""Build libfa2.so (the gfx950 kernels plus the C-ABI host code) in-tree with hipcc.

    python -m exact_attention_62_amd.build          # writes exact_attention_62_amd/libfa2.so
    python -m exact_attention_62_amd.build --sanitize OUT.so
        # host code built with AddressSanitizer and UndefinedBehaviorSanitizer
        # (device code unchanged); load it with the ASan runtime preloaded
        # (sanitizer_runtime() names it) and FA2_LIBRARY=OUT.so

hipcc cross-compiles for gfx950 without a GPU present.  Packed fp32 VALU
instructions are disabled for device code (``-packed-fp32-ops``); the host
pass warns that it does not know that feature, which is harmless.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libfa2.so")

SOURCES = ["fa2_api.cpp", "fa2_fwd_bf16.hip", "fa2_fwd_fp16.hip", "fa2_fwd_f32.hip",
           "fa2_combine.hip", "fa2_bwd.hip", "fa2_decode.hip", "fa2_scratch.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    if not os.path.exists(path):
        path = shutil.which("hipcc") or path
    return path


def common_flags(extra=()):
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-function", f"-I{INCLUDE}", f"-I{CSRC}", *extra]


# Host-only sanitizer flags: each -fsanitize= sits directly after -Xarch_host, so
# that the device pass is built exactly as in the normal library.
SANITIZE_FLAGS = ["-Xarch_host", "-O1", "-Xarch_host", "-g",
                  "-Xarch_host", "-fsanitize=address",
                  "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-fno-sanitize-recover=all",
                  "-Xarch_host", "-fno-omit-frame-pointer"]


def sanitizer_runtime() -> str:
    """The ASan runtime (which carries the UBSan handlers too) of hipcc's clang, to
    preload into a process that loads a sanitized library."""
    import glob
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    found = sorted(glob.glob(os.path.join(rocm, "llvm", "lib", "clang", "*", "lib", "linux",
                                          "libclang_rt.asan-x86_64.so")))
    if not found:
        raise RuntimeError("no libclang_rt.asan-x86_64.so under " + rocm)
    return found[-1]


def build(verbose: bool = False, extra_flags=(), out: str = LIB, sanitize: bool = False) -> str:
    """Compile every source and link the library (libfa2.so, or `out`); returns its path.
    With sanitize, host code is instrumented with ASan + UBSan.  Raises on failure."""
    cc = hipcc()
    if sanitize:
        extra_flags = [*extra_flags, *SANITIZE_FLAGS]
    with tempfile.TemporaryDirectory(prefix="fa2_build_") as tmp:
        cmds, objs = [], []
        for src in SOURCES:
            obj = os.path.join(tmp, os.path.splitext(src)[0] + ".o")
            lang = ["-x", "hip"] if src.endswith(".hip") else []
            cmds.append([cc, *common_flags(extra_flags), *lang, "-c", os.path.join(CSRC, src), "-o", obj])
            objs.append(obj)
        # The sources compile independently; the two forward instantiation
        # files dominate, so they run side by side.
        jobs = max(1, min(len(cmds), int(os.environ.get("MAX_JOBS", "0")) or os.cpu_count() or 1, 8))
        with ThreadPoolExecutor(jobs) as pool:
            for f in [pool.submit(_run, cmd, verbose) for cmd in cmds]:
                f.result()
        tmp_lib = os.path.join(tmp, "libfa2.so")
        link_san = ["-Xarch_host", "-fsanitize=address,undefined"] if sanitize else []
        _run([cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *link_san, *objs, "-o", tmp_lib],
             verbose)
        shutil.copyfile(tmp_lib, out + ".tmp")
        os.replace(out + ".tmp", out)
    return out


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(line for line in r.stdout.splitlines()
                    if "packed-fp32-ops" not in line)  # the host pass's harmless warning
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out, flush=True)


if __name__ == "__main__":
    args = sys.argv[1:]
    if "--sanitize" in args:
        i = args.index("--sanitize")
        print(build(verbose="-v" in args, out=os.path.abspath(args[i + 1]), sanitize=True))
    else:
        print(build(verbose="-v" in args))
