"""Build the gfx950 library libcombine_route_amd.so in-tree with hipcc.

Run as ``python -m combine_route_amd.build`` (or through
``__graft_entry__.build()``); it always recompiles.
"""
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libcombine_route_amd.so")
SOURCES = [os.path.join(PKG, "csrc", f)
           for f in ("ep_plan.cpp", "ep_kernels.hip", "ep_expert.hip", "ep_wire.hip",
                     "ep_standard.hip")]
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    # packed FP32 instructions stay off in the gfx950 code: the compiler would
    # otherwise pair the combine's FP32 adds into v_pk_add_f32. The feature
    # exists only for the device target, so each word of the option goes to
    # the device pass alone (-Xarch_device) and the host pass never sees it.
    *[w for a in ("-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops")
      for w in ("-Xarch_device", a)],
    "-fno-fast-math", "-ffp-contract=off",
    "-Wall", "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"),
    "-I", os.path.join(PKG, "csrc"),
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    return "hipcc"


def build(verbose: bool = False, extra=()) -> str:
    """Compile every source to an object in parallel, then link the library."""
    from concurrent.futures import ThreadPoolExecutor

    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    compile_flags = [f for f in FLAGS if f != "-shared"]

    def compile_one(src):
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        cmd = [hipcc(), *compile_flags, *extra, "-c", "-o", obj, src]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        return obj

    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as pool:
        objs = list(pool.map(compile_one, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
