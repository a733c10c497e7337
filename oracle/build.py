"""Build step for the CPU oracle (test infrastructure): gcc -> oracle/liboracle.so.

-ffp-contract=off keeps every FP32 step a single IEEE operation; no fast-math.
build(sanitize=True, out=path) makes an AddressSanitizer + UndefinedBehavior-
Sanitizer build for the CPU sanitizer test (loaded through SATTN_ORACLE_LIB).
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "sattn_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


SANITIZE = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
            "-fno-omit-frame-pointer"]


def build(verbose: bool = False, sanitize: bool = False, out: str = LIB) -> str:
    opt = SANITIZE if sanitize else ["-O3"]
    cmd = (["gcc", "-std=c11"] + opt + ["-mavx2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-fPIC", "-shared", "-Wall", "-Wextra", "-o", out + ".tmp", SRC, "-lm"])
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
