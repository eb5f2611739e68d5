"""Builds the CPU oracle (test infrastructure) into oracle/liboracle.so with gcc.

Plain C11, double precision, OpenMP over rows.  No fast-math and no FP
contraction, so every operation is the IEEE one the source spells out.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "dsa_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


# AddressSanitizer / UndefinedBehaviorSanitizer build for the CPU tests (load
# it with DSA_ORACLE_LIB and preload gcc's libasan).
SANITIZED_LIB = os.path.join(HERE, "liboracle_sanitized.so")


def build(verbose: bool = False, sanitize: bool = False) -> str:
    out = SANITIZED_LIB if sanitize else LIB
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g"]
    cmd = ["gcc", "-std=c11", "-O2", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off",
           "-Wall", "-Wextra", *(san if sanitize else []), "-o", out + ".tmp", SRC, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    import sys
    print(build(verbose=True, sanitize="--sanitize" in sys.argv))
