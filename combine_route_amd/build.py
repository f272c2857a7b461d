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
                     "ep_standard.hip", "ep_probe.hip", "ep_static.hip")]
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-fno-fast-math", "-ffp-contract=off",
    "-Wall", "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"),
    "-I", os.path.join(PKG, "csrc"),
]
# Packed FP32 instructions stay off in the gfx950 code: the compiler would
# otherwise pair the combine's FP32 adds into v_pk_add_f32. The feature is a
# device feature and is given to the device pass alone: a .hip source is
# compiled twice, once for gfx950 only (to an offload bundle, with this flag)
# and once for the host, which embeds that bundle. build() checks the device
# code it links.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    return "hipcc"


PACKED_FP32 = ("v_pk_add_f32", "v_pk_mul_f32", "v_pk_fma_f32")


def device_code(lib: str = LIB) -> str:
    """Disassembly of the library's gfx950 code: its .hip_fatbin section holds
    one offload bundle per source file, each unbundled and disassembled with
    the ROCm LLVM tools."""
    import re
    import tempfile

    llvm = "/opt/rocm/llvm/bin"
    asm = []
    with tempfile.TemporaryDirectory() as tmp:
        fat = os.path.join(tmp, "fatbin")
        subprocess.run([os.path.join(llvm, "llvm-objcopy"), f"--dump-section=.hip_fatbin={fat}",
                        lib, os.path.join(tmp, "stripped")], check=True)
        with open(fat, "rb") as f:
            data = f.read()
        starts = [m.start() for m in re.finditer(re.escape(b"__CLANG_OFFLOAD_BUNDLE__"), data)]
        for i, beg in enumerate(starts):
            part, co = os.path.join(tmp, f"bundle{i}"), os.path.join(tmp, f"device{i}.co")
            with open(part, "wb") as f:
                f.write(data[beg: starts[i + 1] if i + 1 < len(starts) else len(data)])
            subprocess.run([os.path.join(llvm, "clang-offload-bundler"), "--unbundle",
                            "--type=o", f"--targets=hipv4-amdgcn-amd-amdhsa--{ARCH}",
                            f"--input={part}", f"--output={co}"], check=True)
            asm.append(subprocess.run([os.path.join(llvm, "llvm-objdump"), "-d", co], check=True,
                                      capture_output=True, text=True).stdout)
    return "\n".join(asm)


def device_packed_fp32(lib: str = LIB) -> dict:
    """Packed FP32 instructions in the library's gfx950 code: {mnemonic: count}."""
    import re

    asm = device_code(lib)
    return {m: len(re.findall(rf"\b{m}\b", asm)) for m in PACKED_FP32}


def build(verbose: bool = False, extra=()) -> str:
    """Compile every source to an object in parallel, then link the library."""
    from concurrent.futures import ThreadPoolExecutor

    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    compile_flags = [f for f in FLAGS if f != "-shared"]

    def run(cmd):
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)

    def compile_one(src):
        name = os.path.basename(src)
        obj = os.path.join(objdir, name + ".o")
        if not src.endswith(".hip"):
            run([hipcc(), *compile_flags, *extra, "-c", "-o", obj, src])
            return obj
        fatbin = os.path.join(objdir, name + ".hipfb")
        run([hipcc(), *compile_flags, *DEVICE_FLAGS, *extra, "--offload-device-only", "-c",
             "-o", fatbin, src])
        run([hipcc(), *compile_flags, *extra, "--offload-host-only",
             "-Xclang", "-fcuda-include-gpubinary", "-Xclang", fatbin, "-c", "-o", obj, src])
        return obj

    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as pool:
        objs = list(pool.map(compile_one, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    found = {m: c for m, c in device_packed_fp32(tmp).items() if c}
    if found:
        raise RuntimeError(f"packed FP32 instructions in the gfx950 code: {found}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
