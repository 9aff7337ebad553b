"""Build libmifa.so in-tree with hipcc for gfx950.

Usage: python -m io_aware_softmax_mifa_amd.build [--verbose] [--save-temps DIR]
"""
from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SOURCES = [os.path.join(PKG, "csrc", f) for f in ("mifa_fwd.hip", "mifa_bwd.hip", "mifa_softmax.hip", "mifa_clock.hip")]
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libmifa.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; a ROCm toolchain is required to build libmifa")


def flags(extra=()):
    return [
        f"--offload-arch={ARCH}",
        "-O3",
        "-std=c++20",
        "-fPIC",
        "-shared",
        f"-I{INCLUDE}",
        # Keep the compiler from forming packed fp32 VALU ops (v_pk_mul_f32 and friends).
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        *extra,
    ]


def build_host_asan(out_dir: str, verbose: bool = False) -> str:
    """The same library with AddressSanitizer on the host code only (argument checks, launch
    set-up); the device code is unchanged.  For CPU tests of the C ABI: load it into a process
    started with the ASan runtime preloaded (asan_runtime())."""
    os.makedirs(out_dir, exist_ok=True)
    out = os.path.join(out_dir, "libmifa.so")
    asan = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer", "-shared-libsan"]
    cmd = [hipcc(), *flags(asan), *SOURCES, "-o", out + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, cwd=out_dir, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc (host ASan) failed ({res.returncode}):\n{res.stderr}")
    os.replace(out + ".tmp", out)
    return out


def asan_runtime() -> str:
    """Path of the clang ASan runtime matching hipcc's host compiler."""
    clang = os.path.join(os.path.dirname(os.path.realpath(hipcc())), "..", "lib", "llvm", "bin", "clang")
    for cand in (clang, "/opt/rocm/lib/llvm/bin/clang", shutil.which("clang")):
        if cand and os.path.exists(cand):
            r = subprocess.run([cand, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
            path = r.stdout.strip()
            if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path):
                return path
    raise RuntimeError("clang ASan runtime not found")


def build(verbose: bool = False, save_temps: str | None = None) -> str:
    extra = []
    if save_temps:
        os.makedirs(save_temps, exist_ok=True)
        extra += ["-save-temps", "-Rpass-analysis=kernel-resource-usage"]
    tmp = LIB + f".tmp{os.getpid()}"
    cmd = [hipcc(), *flags(extra), *SOURCES, "-o", tmp]
    cwd = save_temps or PKG
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, cwd=cwd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(line for line in res.stderr.splitlines() if noise not in line)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--verbose", action="store_true")
    ap.add_argument("--save-temps", default=None)
    a = ap.parse_args()
    print(build(verbose=a.verbose, save_temps=a.save_temps))


if __name__ == "__main__":
    main()
