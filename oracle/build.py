"""Build the CPU oracle shared library (test infrastructure only).

gcc, -O2, no fast-math and no floating-point contraction, so that every binary32
operation in the oracle is a single IEEE operation with one rounding.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "kivi_oracle.c")
LIB = os.path.join(HERE, "libkivi_oracle.so")


def build(verbose: bool = False, out: str = LIB, extra_flags=()) -> str:
    """``extra_flags`` go after the standard ones, e.g. sanitizer options for a checked
    build written to another path (``out``)."""
    cmd = [
        "gcc", "-std=c11", "-O2", "-fPIC", "-shared",
        "-ffp-contract=off", "-fno-fast-math", "-fexcess-precision=standard",
        "-Wall", "-Wextra", "-Wno-unused-parameter", *extra_flags,
        SRC, "-o", out + ".tmp", "-lm",
    ]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
