"""Build the CPU oracle library (plain C, gcc) in place: oracle/liboracle.so.

Test infrastructure: the library it builds is only loaded by the test suite,
the package smoke check and the benchmark's CPU-baseline leg.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

# No fast-math, no FMA contraction: the dequantisation step must be the exact
# product rounded once to binary32, and the attention sums are plain binary64.
CFLAGS = ["-O2", "-std=gnu11", "-fPIC", "-shared", "-fno-fast-math",
          "-ffp-contract=off", "-Wall", "-Wextra", "-Werror"]


def build(verbose=False):
    cmd = ["gcc", *CFLAGS, "-o", LIB + ".tmp", SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


def build_sanitized(out, verbose=False):
    """The same library built with AddressSanitizer and UndefinedBehaviorSanitizer
    (any report aborts), at `out`. Load it into a process that has the ASan
    runtime preloaded (LD_PRELOAD), with HP_ORACLE_LIB=out."""
    flags = [f for f in CFLAGS if f != "-O2"] + [
        "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
        "-fno-sanitize-recover=all"]
    cmd = ["gcc", *flags, "-o", out, SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
