"""Build the CPU oracle (test infrastructure only) with gcc.

Two shared libraries come from oracle.c: liboracle_f32.so stores tensors in
float (the pages' single precision) and liboracle_f64.so stores them in double
(for finite-difference checks).  Both accumulate every sum in double and are
built with -ffp-contract=off, so each statement of the update rules rounds
once.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
TARGETS = {
    "liboracle_f32.so": [],
    "liboracle_f64.so": ["-DOR_REAL=double", "-DOR_REAL_IS_DOUBLE"],
}


def build(verbose=False):
    for name, defs in TARGETS.items():
        out = os.path.join(HERE, name)
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
               "-fno-fast-math", "-Wall", "-Wno-unknown-pragmas", *defs, SRC, "-o", out + ".tmp", "-lm"]
        if verbose:
            print(" ".join(cmd))
        subprocess.check_call(cmd)
        os.replace(out + ".tmp", out)


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
