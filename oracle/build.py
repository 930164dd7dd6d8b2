"""Build step for the C oracle (test infrastructure; see msd_oracle.c).

Compiled with -O2 -ffp-contract=off and without -ffast-math so that every
fp32 operation is rounded exactly once, in source order.
"""
from __future__ import annotations

import os
import subprocess

_HERE = os.path.dirname(os.path.abspath(__file__))


def build(verbose: bool = False) -> str:
    src = os.path.join(_HERE, "msd_oracle.c")
    out = os.path.join(_HERE, "libmsd_oracle.so")
    tmp = out + ".tmp"
    cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
           "-std=c11", "-Wall", "-Wextra", "-shared", "-fPIC", src, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build_sanitized(verbose: bool = False) -> str:
    """The same oracle built with AddressSanitizer and UndefinedBehaviorSanitizer
    (gcc; any report aborts), for running the oracle's pins under them.  The
    process that loads it must preload gcc's libasan."""
    src = os.path.join(_HERE, "msd_oracle.c")
    out = os.path.join(_HERE, "libmsd_oracle_san.so")
    tmp = out + ".tmp"
    cmd = ["gcc", "-O1", "-g", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
           "-std=c11", "-Wall", "-Wextra", "-shared", "-fPIC", src, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
