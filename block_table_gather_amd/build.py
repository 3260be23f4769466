"""Build libhp.so (the C-ABI library of include/hp.h) for gfx950, in place.

    python block_table_gather_amd/build.py [-v] [-DNAME=VALUE ...] [-o OUT]

Run it as a script (or load it by path): importing the package would load the
library this builds.

Extra -D definitions (HP_GATHER_UNIT_BYTES, HP_THREADS, ...) override the build
time tuning knobs; -o writes the library elsewhere (used for tuning sweeps).
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
SOURCES = [os.path.join(CSRC, "hp_api.cpp"), os.path.join(CSRC, "hp_kernels.hip"),
           os.path.join(CSRC, "hp_attention.hip")]
LIB = os.path.join(HERE, "libhp.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    # packed fp32 instructions stay off: the code relies on ordinary fp32 ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
    "-I", CSRC,
]


def build(verbose=False, defines=(), out=None):
    """Compile every source to an object in parallel, then link the library."""
    out = out or LIB
    tmp = out + ".tmp"
    objs = [f"{tmp}.{os.path.basename(src)}.o" for src in SOURCES]
    compile_flags = [f for f in FLAGS if f != "-shared"]
    procs = []
    for src, obj in zip(SOURCES, objs):
        cmd = [HIPCC, *compile_flags, *defines, "-c", "-x", "hip", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((cmd, subprocess.Popen(cmd)))
    failed = [cmd for cmd, p in procs if p.wait() != 0]
    try:
        if failed:
            raise subprocess.CalledProcessError(1, failed[0])
        link = [HIPCC, "--offload-arch=gfx950", "-fPIC", "-shared", *objs, "-o", tmp]
        if verbose:
            print(" ".join(link), flush=True)
        subprocess.run(link, check=True)
    finally:
        for obj in objs:
            if os.path.exists(obj):
                os.remove(obj)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    args = sys.argv[1:]
    out = None
    if "-o" in args:
        i = args.index("-o")
        out = args[i + 1]
        del args[i: i + 2]
    defs = [a for a in args if a.startswith("-D")]
    print(build(verbose="-v" in args, defines=defs, out=out))
