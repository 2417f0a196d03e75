"""Build libbqmoe.so (gfx950 HIP kernels + C ABI) in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libbqmoe.so")
# roofline ceilings (read stream, matrix-core peak), a library of their own
CEIL_SOURCES = ["ceilings.hip"]
CEIL_LIB = os.path.join(HERE, "libbqceil.so")

SOURCES = ["pack.cpp", "api.cpp", "route.hip", "decode.hip", "prefill.hip", "prefill16.hip",
           "prefill2x.hip", "noalloc.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# Packed fp32 VALU forms are switched off for every kernel: the scalar forms
# are used throughout.
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-result",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


# The decode kernels keep matrix-core results in ordinary vector registers:
# their epilogue per op is a single multiply-add, which would otherwise need
# an extra accumulator-register read each.
EXTRA = {"decode.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def compile_command(src: str, out: str, device_asm: bool = False) -> list:
    """hipcc command line for one source (an object file, or device assembly)."""
    path = os.path.join(CSRC, src)
    if src.endswith(".hip"):
        mode = ["--cuda-device-only", "-S"] if device_asm else ["-c"]
        return [HIPCC, "-x", "hip", f"--offload-arch={ARCH}", *COMMON, *EXTRA.get(src, []),
                *mode, path, "-o", out]
    return [HIPCC, "-x", "c++", *COMMON, "-c", path, "-o", out]


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, src + ".o")
    cmd = compile_command(src, obj)
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = (r.stdout + r.stderr).splitlines()
    # the host pass does not know the device-only feature flag: not an error
    out = [l for l in out if "packed-fp32-ops" not in l or "error" in l]
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n" + "\n".join(out))
    if verbose and out:
        print("\n".join(out))
    return obj


def _link(objs: list, lib: str, verbose: bool) -> None:
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    """Compile every source for gfx950 and link libbqmoe.so and libbqceil.so.
    Always recompiles."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + CEIL_SOURCES
    with ThreadPoolExecutor(max_workers=min(len(srcs), os.cpu_count() or 4)) as ex:
        objs = dict(zip(srcs, ex.map(lambda s: _compile(s, verbose), srcs)))
    _link([objs[s] for s in SOURCES], LIB, verbose)
    _link([objs[s] for s in CEIL_SOURCES], CEIL_LIB, verbose)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
    print(LIB)
