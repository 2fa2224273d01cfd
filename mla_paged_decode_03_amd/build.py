"""Builds libmla_decode.so (HIP for gfx950) in-tree.

Usage: python -m mla_paged_decode_03_amd.build [-v]
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libmla_decode.so")
BUILD = os.path.join(PKG, "_build")
SOURCES = ["plan.cpp", "abi.hip", "decode.hip", "merge.hip", "gemm.hip", "quant.hip", "cache_write.hip", "prefill.hip", "bmm8.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANGXX = "/opt/rocm/lib/llvm/bin/clang++"
ARCH = "gfx950"

COMMON = [
    "-O3", "-std=c++20", "-fPIC", "-Wall", "-Wno-unused-function",
    # Packed fp32 VALU ops stay off: the compiler must not form v_pk_*_f32.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _compile(src: str, verbose: bool, extra) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    path = os.path.join(CSRC, src)
    if src.endswith(".cpp"):
        cmd = [HIPCC, "-x", "c++", "-O3", "-std=c++17", "-fPIC", "-Wall", "-c", path, "-o", obj]
    else:
        cmd = [HIPCC, f"--offload-arch={ARCH}", *COMMON, *extra, "-c", path, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    msg = "\n".join(x for x in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in x)  # host pass does not know the feature
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {src}\n{msg}")
    if verbose and msg.strip():
        print(msg)
    return obj


def _hip_runtime_link_args():
    """Link against the HIP runtime that torch loads, when torch is installed.

    torch ships its own libamdhip64.so (without a SONAME).  A library linked to
    ROCm's libamdhip64.so.7 would bring a second HIP runtime into the process,
    and the two do not share devices, streams or allocations.  Linking to
    torch's copy by path (with a RUNPATH to its directory) makes the dynamic
    linker reuse the runtime torch already loaded.
    """
    try:
        import importlib.util
        spec = importlib.util.find_spec("torch")
        if spec and spec.origin:
            lib_dir = os.path.join(os.path.dirname(spec.origin), "lib")
            hip = os.path.join(lib_dir, "libamdhip64.so")
            if os.path.exists(hip):
                return [f"-L{lib_dir}", "-l:libamdhip64.so", f"-Wl,-rpath,{lib_dir}", "-Wl,--disable-new-dtags"]
    except Exception:
        pass
    return ["-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"]


def build(verbose: bool = False, extra=()) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, list(extra)), SOURCES))
    tmp = OUT + ".tmp"
    # Plain clang++ link (the objects already carry their gfx950 code objects), so
    # that no HIP runtime other than the one chosen below is pulled in.
    cmd = [CLANGXX, "-shared", "-fPIC", *objs, "-o", tmp, *_hip_runtime_link_args()]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed\n" + r.stdout + r.stderr)
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    v = "-v" in sys.argv
    extra = [a for a in sys.argv[1:] if a != "-v"]
    print(build(verbose=v, extra=extra))
