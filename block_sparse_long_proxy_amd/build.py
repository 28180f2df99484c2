"""Build libpxa.so (the HIP kernels + C ABI) in-tree for gfx950.

    python -m block_sparse_long_proxy_amd.build [--verbose] [--save-temps] [--sanitize]

Every source under csrc/ is compiled with hipcc to an object in _build/ and
linked into block_sparse_long_proxy_amd/libpxa.so.  Always recompiles.

--sanitize builds block_sparse_long_proxy_amd/libpxa_san.so instead: the same
sources with AddressSanitizer and UndefinedBehaviorSanitizer on the host code
only (the device code is built as usual), for running the host-side tests of
the C ABI's validation paths under the sanitizers (load the ASan runtime first,
see asan_runtime()).
"""
from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libpxa.so")
SAN_LIB = os.path.join(PKG, "libpxa_san.so")
ARCH = "gfx950"
# host code only: each -fsanitize= applies to the host pass (-Xarch_host)
SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
            "-Xarch_host", "-g"]

COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
    # keep the compiler from emitting packed fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result", "-I", os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libpxa.so)")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def asan_runtime() -> str:
    """Path of the compiler's AddressSanitizer runtime (to LD_PRELOAD into a
    process that loads libpxa_san.so)."""
    clang = os.path.join(os.path.dirname(os.path.realpath(hipcc())), "..", "lib", "llvm", "bin", "clang")
    for c in (clang, "/opt/rocm/llvm/bin/clang"):
        if os.path.exists(c):
            r = subprocess.run([c, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                               text=True)
            path = r.stdout.strip()
            if r.returncode == 0 and os.path.exists(path):
                return path
    raise RuntimeError("AddressSanitizer runtime not found")


def _compile(src: str, save_temps: bool, verbose: bool, sanitize: bool = False) -> str:
    obj = os.path.join(BUILD, ("san_" if sanitize else "") + os.path.basename(src) + ".o")
    cmd = [hipcc()] + COMMON + (SANITIZE if sanitize else []) + ["-c", src, "-o", obj]
    if save_temps:
        cmd += ["-save-temps=obj"]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(line for line in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in line)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {os.path.basename(src)}:\n{out}")
    if verbose and out.strip():
        print(out, file=sys.stderr)
    return obj


def build(verbose: bool = False, save_temps: bool = False, sanitize: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    with ThreadPoolExecutor(min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, save_temps, verbose, sanitize), srcs))
    lib = SAN_LIB if sanitize else LIB
    tmp = lib + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    if sanitize:
        cmd[1:1] = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                    "-shared-libsan"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, lib)
    return lib


def main() -> None:
    ap = argparse.ArgumentParser()
    ap.add_argument("--verbose", action="store_true")
    ap.add_argument("--save-temps", action="store_true")
    ap.add_argument("--sanitize", action="store_true",
                    help="build libpxa_san.so with ASan/UBSan on the host code")
    a = ap.parse_args()
    print(build(a.verbose, a.save_temps, a.sanitize))


if __name__ == "__main__":
    main()
