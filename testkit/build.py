"""Build step for the seeded input generator: gcc -> testkit/libsattn_testkit.so."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "sattn_testkit.c")
LIB = os.path.join(HERE, "libsattn_testkit.so")


SANITIZE = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
            "-fno-omit-frame-pointer"]


def build(verbose: bool = False, sanitize: bool = False, out: str = LIB) -> str:
    """sanitize=True: AddressSanitizer + UndefinedBehaviorSanitizer build at
    `out` (loaded through SATTN_TESTKIT_LIB by the CPU sanitizer test)."""
    opt = SANITIZE if sanitize else ["-O2"]
    cmd = (["gcc", "-std=c11"] + opt + ["-fopenmp", "-ffp-contract=off", "-fPIC", "-shared",
           "-Wall", "-Wextra", "-o", out + ".tmp", SRC, "-lm"])
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
